"""GPU parity of the grouped A4W4 GEMM over MoE experts (expert weights and activations
in OCP MXFP4: "Kimi-K3-Quark-MXFP4-AttnFP8", section "Model Quantization"), through the
C ABI, against the oracle's exact GEMM applied group by group:
|gpu - exact| <= 2^-8 |exact| + 1e-6 sum|a w| per element.

Group e multiplies the packed activation rows offsets[e] .. offsets[e+1]-1 with expert
weight e.  The pages give no expert shapes; these are synthetic: empty groups, single
rows, ragged sizes from 1 to 1000 rows (above the bound the caller passes as well), ragged
N, K = 2048 (128-column tiles) and above (the grouped decode ring), both scale-row sizes
(K <= 8192 and K = 10240).
"""
import numpy as np
import pytest

from block_scaled_precision_act_amd import synth
from parity import bf16_host, gemm_within_tolerance, to_dev

pytestmark = pytest.mark.gpu
NT = 16


def _grouped_case(orc, seed, sizes, N, K):
    G, T = len(sizes), int(sum(sizes))
    x = synth.f64_to_bf16_bits(synth.normal(seed, max(T, 1) * K)).reshape(max(T, 1), K)[:T]
    w = synth.weight_normal(seed + 1, G * N, K, 0.02)
    qa, sa = orc.mx_quant_bf16(np.ascontiguousarray(x), nthreads=NT)
    qw, sw = orc.mx_quant_f32(w, nthreads=NT)
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    return qa, sa, qw.reshape(G, N, K // 2), sw.reshape(G, N, K // 32), offsets


@pytest.mark.parametrize("sizes,N,K,max_rows", [
    ([0, 1, 17, 32, 0, 5], 512, 2048, 32),          # K = 2048: 128-column tiles, 32-row chunks, empty groups
    ([40, 3, 64, 0, 9], 1000, 2048, 64),            # K = 2048, 64-row chunks, ragged N
    ([64, 33, 0, 40, 2], 300, 4096, 64),            # 64-row kernel, ragged N
    ([3, 64, 1], 1000, 10240, 64),                  # K > 8192 (512-byte scale rows)
    ([9, 0, 30], 96, 10240, 32),
    ([0, 7, 32, 19], 640, 7168, 32),                # K % 2048 != 0 (an up / gate projection's K): the
    ([40, 2, 64], 300, 7168, 64),                   #   LDS-staged decode kernel, 32- and 64-row chunks
    ([5, 33], 200, 512, 64),                        # one 512-K stage
    ([3, 0, 12], 100, 1536, 32),
    ([1, 2, 0, 3] * 8, 4096, 4096, 32),             # 32 experts x 32 tiles: 128-column tiles, K in 4 parts
])
def test_grouped_a4w4_matches_oracle(mx, orc, sizes, N, K, max_rows):
    import torch
    qa, sa, qw, sw, offsets = _grouped_case(orc, 7 * N + K + len(sizes), sizes, N, K)
    T = int(offsets[-1])
    y = torch.full((T, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    mx.gemm_a4w4_grouped(to_dev(qa), to_dev(sa), to_dev(qw), to_dev(sw), to_dev(offsets), max_rows, y=y)
    yh = bf16_host(y)
    for e in range(len(sizes)):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r0 == r1:
            continue
        ye, ad, _ = orc.gemm_a4w4_at(qa[r0:r1], sa[r0:r1], qw[e], sw[e], nthreads=NT)
        ok, ratio, nbad = gemm_within_tolerance(yh[r0:r1], ye, ad)
        print("group %d (%d rows): max err/bound %.4f" % (e, r1 - r0, ratio))
        assert ok, "group %d: %d elements outside tolerance (max err/bound %.3g)" % (e, nbad, ratio)


@pytest.mark.parametrize("sizes,N,K,max_rows", [
    ([100, 0, 65, 7], 512, 2048, 32),        # groups above the bound: 32-row chunks, every row written
    ([300, 1000, 3], 256, 4096, 64),         # prefill-sized groups in 64-row chunks
    ([64, 65, 128, 129], 300, 2048, 1),      # chunk edges; a bound far below the real sizes
    ([200, 0, 129, 1], 640, 2048, 64),       # K = 2048 in 64-row chunks, groups above the bound
    ([130, 0, 65], 256, 7168, 32),           # K % 2048 != 0 in 32-row chunks, groups above the bound
    ([100, 129], 128, 1536, 64),
])
def test_grouped_every_row_of_large_groups(mx, orc, sizes, N, K, max_rows):
    """max_rows only picks 32- or 64-row chunks: groups of 65 .. 1000 rows, and groups larger than the
    bound the caller passed, are computed in full (checked against the oracle group by group)."""
    import torch
    qa, sa, qw, sw, offsets = _grouped_case(orc, 3 * N + K + sum(sizes), sizes, N, K)
    T = int(offsets[-1])
    y = torch.full((T, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    mx.gemm_a4w4_grouped(to_dev(qa), to_dev(sa), to_dev(qw), to_dev(sw), to_dev(offsets), max_rows, y=y)
    yh = bf16_host(y)
    for e in range(len(sizes)):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r0 == r1:
            continue
        ye, ad, _ = orc.gemm_a4w4_at(qa[r0:r1], sa[r0:r1], qw[e], sw[e], nthreads=NT)
        ok, ratio, nbad = gemm_within_tolerance(yh[r0:r1], ye, ad)
        print("group %d (%d rows, max_rows %d): max err/bound %.4f" % (e, r1 - r0, max_rows, ratio))
        assert ok, "group %d: %d elements outside tolerance (max err/bound %.3g)" % (e, nbad, ratio)


@pytest.mark.parametrize("K", [4096, 8192, 7168])
def test_grouped_equals_per_group_gemm_bit_for_bit(mx, orc, K):
    # above K = 2048 every grouped kernel (the decode ring, the LDS-staged kernel, or 128-column tiles walking
    # K in parts) sums each output in the K order of the ungrouped decode kernels these groups take: each
    # group's rows come out identical to mx_gemm_a4w4_bf16 on that group alone (here: 20 tile workgroups and
    # 32-row chunks, so K = 4096 and 8192 take the ring and K = 7168 the tiles).
    import torch
    sizes, N = [5, 0, 20, 11], 640
    qa, sa, qw, sw, offsets = _grouped_case(orc, 99, sizes, N, K)
    yg = mx.gemm_a4w4_grouped(to_dev(qa), to_dev(sa), to_dev(qw), to_dev(sw), to_dev(offsets), 32)
    for e in range(len(sizes)):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r0 == r1:
            continue
        ys = mx.gemm_a4w4(to_dev(qa[r0:r1]), to_dev(sa[r0:r1]), to_dev(qw[e]), to_dev(sw[e]))
        assert torch.equal(yg[r0:r1].view(torch.int16), ys.view(torch.int16)), "group %d differs" % e


def test_grouped_k2048_chunk_sizes_agree_bit_for_bit(mx, orc):
    # at K = 2048 both chunk sizes (max_rows <= 32: 32-row chunks, else 64) sum every output in the same
    # K order, one 32-row fragment at a time: the results are identical
    import torch
    sizes, N = [70, 0, 33, 5, 31], 900
    qa, sa, qw, sw, offsets = _grouped_case(orc, 1234, sizes, N, 2048)
    args = (to_dev(qa), to_dev(sa), to_dev(qw), to_dev(sw), to_dev(offsets))
    y32 = mx.gemm_a4w4_grouped(*args, 32)
    y64 = mx.gemm_a4w4_grouped(*args, 64)
    assert torch.equal(y32.view(torch.int16), y64.view(torch.int16))
