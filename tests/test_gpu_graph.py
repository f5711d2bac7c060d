"""The entry points enqueue only kernels (no allocation, no memset, no host sync), so a
whole layer can be captured into a HIP graph.  Each replay, with eager work and host
synchronizations in between, must reproduce the eager result bit for bit."""
import numpy as np
import pytest

from block_scaled_precision_act_amd import synth
from parity import bf16_dev

pytestmark = pytest.mark.gpu


def _replays_match(mx, torch, thunk, outs):
    thunk()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        thunk()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        thunk()
    for rep in range(4):
        for o in outs:
            o.zero_()
        junk = torch.randn(1 << 20, device="cuda").sum()  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o.view(torch.uint8), e.view(torch.uint8)), "replay %d differs" % rep
        del junk


# decode rings (64, 16 rows), the 128-row tile with copy and MFMA waves (300), the 256 x 224 tile (1300 x 7000),
# the split-K decode kernel (64 x 7168 x 8192) and the 128-row tile with K in two parts (256 x 2048 x 8192)
@pytest.mark.parametrize("M,N,K", [(64, 512, 1024), (300, 512, 1024), (64, 7168, 8192), (16, 2000, 4096),
                                   (1300, 7000, 512), (256, 2048, 8192)])
def test_a4w4_layer_graph_replay(mx, M, N, K):
    import torch
    x = bf16_dev(synth.act_normal(61, M, K))
    qw, sw = mx.quant_weight_mx(torch.from_numpy(synth.weight_normal(62, N, K, 0.02)).cuda())
    qa = torch.empty((M, K // 2), dtype=torch.uint8, device="cuda")
    sa = torch.empty((M, K // 32), dtype=torch.uint8, device="cuda")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    wsb = mx.mx_gemm_a4w4_workspace_bytes(M, N, K)
    ws = torch.zeros(max(wsb, 16), dtype=torch.uint8, device="cuda")  # zero-filled before first use

    def layer():
        s = torch.cuda.current_stream().cuda_stream
        assert mx.mx_quant_act_bf16(x.data_ptr(), M, K, qa.data_ptr(), sa.data_ptr(), s) == 0
        assert mx.mx_gemm_a4w4_bf16(qa.data_ptr(), sa.data_ptr(), qw.data_ptr(), sw.data_ptr(), y.data_ptr(),
                                    M, N, K, ws.data_ptr(), wsb, s) == 0

    _replays_match(mx, torch, layer, [qa, sa, y])


# the one-call layer: one launch that quantizes inside the split-K GEMM (M <= 8), and quantizer + GEMM in one
# call (M = 64), each with its workspace shared by the replays
@pytest.mark.parametrize("M,N,K", [(1, 7168, 8192), (8, 2048, 16384), (64, 7168, 8192)])
def test_a4w4_one_call_layer_graph_replay(mx, M, N, K):
    import torch
    x = bf16_dev(synth.act_normal(71, M, K))
    qw, sw = mx.quant_weight_mx(torch.from_numpy(synth.weight_normal(72, N, K, 0.02)).cuda())
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    wsb = mx.mx_linear_a4w4_workspace_bytes(M, N, K)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")  # zero-filled before first use

    def layer():
        s = torch.cuda.current_stream().cuda_stream
        assert mx.mx_linear_a4w4_bf16(x.data_ptr(), qw.data_ptr(), sw.data_ptr(), y.data_ptr(), M, N, K,
                                      ws.data_ptr(), wsb, s) == 0

    _replays_match(mx, torch, layer, [y])
    assert int(ws[:8 << 20].count_nonzero()) == 0  # the partial area is left zero by every replay


# the allocation-free GEMM, for callers under graph capture: its split-K workspace is the library's static
# per-GPU array, left zero by every replay
@pytest.mark.parametrize("M,N,K", [(64, 7168, 8192), (256, 2048, 8192)])
def test_a4w4_noalloc_graph_replay(mx, M, N, K):
    import torch
    assert mx.mx_gemm_a4w4_workspace_bytes(M, N, K) > 0, "the shape should take a split-K plan"
    qa, sa = mx.quant_act_mx(bf16_dev(synth.act_normal(81, M, K)))
    qw, sw = mx.quant_weight_mx(torch.from_numpy(synth.weight_normal(82, N, K, 0.02)).cuda())
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def gemm():
        s = torch.cuda.current_stream().cuda_stream
        assert mx.mx_gemm_a4w4_bf16_noalloc(qa.data_ptr(), sa.data_ptr(), qw.data_ptr(), sw.data_ptr(), y.data_ptr(),
                                            M, N, K, s) == 0

    _replays_match(mx, torch, gemm, [y])
    assert torch.equal(y.view(torch.int16), mx.gemm_a4w4(qa, sa, qw, sw).view(torch.int16))


# the decode ring (64 x 512 x 1024), the split-K kernel (64 x 4096 x 8192), the 128-row FP8 tile with copy and
# MFMA waves (300 x 512 x 1024), in two K parts (256 x 2048 x 8192), and the 256 x 224 FP8 tile (2200 x 3900 x 512)
@pytest.mark.parametrize("M,N,K", [(64, 512, 1024), (64, 4096, 8192), (300, 512, 1024), (256, 2048, 8192),
                                   (2200, 3900, 512)])
def test_a8w8_layer_graph_replay(mx, M, N, K):
    import torch
    x = bf16_dev(synth.act_normal(63, M, K))
    qw, sw = mx.quant_weight_ptpc(torch.from_numpy(synth.weight_normal(64, N, K, 0.01)).cuda())
    qa = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    sa = torch.empty((M,), dtype=torch.float32, device="cuda")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    wsb = mx.gemm_a8w8_ptpc_workspace_bytes(M, N, K)
    assert (wsb > 0) == (K == 8192)
    ws = torch.zeros(max(wsb, 256), dtype=torch.uint8, device="cuda")

    def layer():
        s = torch.cuda.current_stream().cuda_stream
        assert mx.ptpc_quant_act_fp8(x.data_ptr(), M, K, qa.data_ptr(), sa.data_ptr(), s) == 0
        assert mx.gemm_a8w8_ptpc_bf16(qa.data_ptr(), sa.data_ptr(), qw.data_ptr(), sw.data_ptr(), y.data_ptr(),
                                      M, N, K, ws.data_ptr(), wsb, s) == 0

    _replays_match(mx, torch, layer, [qa, sa, y])


def test_a4w4_grouped_graph_replay(mx):
    # the grouped MoE GEMM reads its group offsets on the device: capturable with routing on the GPU
    import torch
    sizes, N, K = [3, 0, 17, 40], 512, 2048
    G, T = len(sizes), sum(sizes)
    x = bf16_dev(synth.act_normal(65, T, K))
    qw, sw = mx.quant_weight_mx(torch.from_numpy(synth.weight_normal(66, G * N, K, 0.02)).cuda())
    qw, sw = qw.view(G, N, K // 2), sw.view(G, N, K // 32)
    offsets = torch.tensor([0] + list(np.cumsum(sizes)), dtype=torch.int32, device="cuda")
    qa = torch.empty((T, K // 2), dtype=torch.uint8, device="cuda")
    sa = torch.empty((T, K // 32), dtype=torch.uint8, device="cuda")
    y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")

    def layer():
        s = torch.cuda.current_stream().cuda_stream
        assert mx.mx_quant_act_bf16(x.data_ptr(), T, K, qa.data_ptr(), sa.data_ptr(), s) == 0
        assert mx.mx_gemm_a4w4_grouped_bf16(qa.data_ptr(), sa.data_ptr(), qw.data_ptr(), sw.data_ptr(), y.data_ptr(),
                                            offsets.data_ptr(), G, 64, N, K, s) == 0

    _replays_match(mx, torch, layer, [qa, sa, y])
