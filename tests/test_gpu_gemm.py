"""GPU parity of the A4W4 and A8W8 GEMMs: HIP kernels (through the C ABI) vs the
oracle's exact result, within |gpu - exact| <= 2^-8 |exact| + 1e-6 sum|a w|.

Layer: Y = X . W^T, W stored (out, in) ("Kimi-K3 DSpark O-Proj-only MXFP4",
section "Exact quantization coverage"); A8W8 scheme of "Kimi-K3-DSpark-FP8-PTPC",
section "Phase 1 FP8 PTPC Quantization".  The GEMM inputs are quantized by the
oracle, so these tests isolate the GEMM kernels; the layer tests at the end run
the HIP quantizer in front of the HIP GEMM.
"""
import functools

import numpy as np
import pytest

from block_scaled_precision_act_amd import synth
from parity import bf16_dev, bf16_host, gemm_within_tolerance, to_dev

pytestmark = pytest.mark.gpu
NT = 16  # oracle threads


@functools.lru_cache(maxsize=None)
def _weight_mx(name):
    import oracle
    w = synth.make_weight(synth.CONFIGS[name])
    return oracle.mx_quant_f32(w, nthreads=NT)


@functools.lru_cache(maxsize=None)
def _weight_ptpc(name):
    import oracle
    w = synth.make_weight(synth.CONFIGS[name])
    return oracle.ptpc_quant_f32(w, nthreads=NT)


def _check(y_gpu, y, ad, what):
    ok, ratio, nbad = gemm_within_tolerance(y_gpu, y, ad)
    print("%s: max err/bound %.4f" % (what, ratio))
    assert ok, "%s: %d elements outside tolerance (max err/bound %.3g)" % (what, nbad, ratio)


def _a4w4_gpu(mx, qa, sa, qw, sw):
    return bf16_host(mx.gemm_a4w4(to_dev(qa), to_dev(sa), to_dev(qw), to_dev(sw)))


def _a8w8_gpu(mx, qa, sa, qw, sw):
    return bf16_host(mx.gemm_a8w8(to_dev(qa), to_dev(sa), to_dev(qw), to_dev(sw)))


def _random_mx(orc, seed, M, N, K, w_std=0.02):
    x = synth.f64_to_bf16_bits(synth.normal(seed, M * K)).reshape(M, K)
    w = synth.weight_normal(seed + 1, N, K, w_std)
    qa, sa = orc.mx_quant_bf16(x, nthreads=NT)
    qw, sw = orc.mx_quant_f32(w, nthreads=NT)
    return qa, sa, qw, sw


# Decode paths: M <= 64 with K % 2048 == 0 (scale rows up to 256 or up to 512 bytes) and not; M <= 128 in two
# 64-row halves (K % 2048 == 0, K <= 8192) and not.
# Tile paths (M > 128): K % 512, % 256 or neither; 128-row tiles when there would be at most 160 tiles of
# 256 rows, else 256 x 224 tiles when they take fewer rounds (1300 x 7000, 2600 x 4001, the prefill and
# M = 2048 configurations), else 256 x 256.  Ragged M and N, several tiles.
# A8W8 runs the same shapes: decode ring for M <= 64 with K % 512 == 0, tile kernel for K % 512 == 0.
SHAPES = [(1, 256, 128), (3, 100, 384), (16, 7168, 1024), (17, 33, 256), (37, 1000, 1024), (64, 512, 512),
          (100, 300, 2048), (128, 1024, 8192), (129, 300, 384), (300, 700, 1024), (512, 512, 512),
          (600, 1100, 2176), (257, 257, 128), (259, 1030, 256), (1000, 800, 4096), (777, 520, 768),
          (1, 256, 2048), (33, 520, 4096), (64, 100, 2048), (7, 300, 16384), (48, 77, 6144),
          (2200, 3896, 512), (2200, 3900, 1024), (40, 129, 16384), (64, 96, 10240),
          (1300, 7000, 512), (2600, 4001, 512), (65, 520, 4096), (127, 1000, 8192), (96, 77, 2048),
          # the 512-K LDS-staged decode kernel at 17..32 and 65..128 rows (K % 2048 != 0, or K > 8192), and
          # the register-staged decode kernel at 33..64 and 65..128 rows (K % 512 != 0), e.g. a 7168-wide input
          (24, 300, 7168), (100, 300, 7168), (100, 77, 10240), (48, 100, 384), (100, 100, 640),
          # the decode rings at the o_proj width where no split-K plan applies (2 or 3 parts of 2048)
          (64, 7168, 4096), (1, 7168, 6144)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_a4w4_shapes(mx, orc, M, N, K):
    qa, sa, qw, sw = _random_mx(orc, M * 7 + N + K, M, N, K)
    y, ad, _ = orc.gemm_a4w4_at(qa, sa, qw, sw, nthreads=NT)
    _check(_a4w4_gpu(mx, qa, sa, qw, sw), y, ad, "a4w4 %dx%dx%d" % (M, N, K))


@pytest.mark.parametrize("M,N,K", [(300, 520, 1024), (260, 300, 512)])
def test_a4w4_scales_4byte_aligned(mx, orc, M, N, K):
    # scale rows only 4-byte aligned (allowed by the ABI): the tile path must not use 16-byte scale copies
    import torch
    qa, sa, qw, sw = _random_mx(orc, M + N + K + 1, M, N, K)
    y, ad, _ = orc.gemm_a4w4_at(qa, sa, qw, sw, nthreads=NT)

    def shifted(a):
        buf = torch.zeros(a.size + 4, dtype=torch.uint8, device="cuda")
        view = buf[4:].view(a.shape)
        view.copy_(torch.from_numpy(a))
        assert view.data_ptr() % 16 != 0
        return view

    out = mx.gemm_a4w4(to_dev(qa), shifted(sa), to_dev(qw), shifted(sw))
    _check(bf16_host(out), y, ad, "a4w4 4-byte-aligned scales %dx%dx%d" % (M, N, K))


def test_a4w4_tiny_config_full(mx, orc):
    cfg = synth.CONFIGS["tiny_a4w4"]
    qw, sw = _weight_mx("tiny_a4w4")
    qa, sa = orc.mx_quant_bf16(synth.make_activations(cfg))
    y, ad, _ = orc.gemm_a4w4_at(qa, sa, qw, sw)
    _check(_a4w4_gpu(mx, qa, sa, qw, sw), y, ad, "tiny 8x256x512")


def test_a4w4_decode_config_full(mx, orc):
    cfg = synth.CONFIGS["oproj_decode_a4w4"]
    qw, sw = _weight_mx("oproj_decode_a4w4")
    qa, sa = orc.mx_quant_bf16(synth.make_activations(cfg))
    y, ad, _ = orc.gemm_a4w4_at(qa, sa, qw, sw, nthreads=NT)
    _check(_a4w4_gpu(mx, qa, sa, qw, sw), y, ad, "o_proj decode 64x7168x8192")


def _sample(n, k, seed):
    rng = np.random.default_rng(seed)
    pick = set(range(min(n, 16))) | set(range(max(0, n - 16), n)) | set(rng.choice(n, min(n, k), replace=False).tolist())
    return np.array(sorted(pick), np.int64)


def _sampled_check(mx, orc, qa, sa, qw, sw, what, seed, gemm="a4w4", sa_scales=None):
    M, N = qa.shape[0], qw.shape[0]
    yg = (_a4w4_gpu if gemm == "a4w4" else _a8w8_gpu)(mx, qa, sa, qw, sw)
    rows, cols = _sample(M, 96, seed), _sample(N, 48, seed + 1)
    f = orc.gemm_a4w4_at if gemm == "a4w4" else orc.gemm_a8w8_at
    y, ad = f(qa, sa, qw, sw, rows=rows, nthreads=NT)[:2]
    _check(yg[rows], y, ad, what + " (sampled rows, all columns)")
    y, ad = f(qa, sa, qw, sw, cols=cols, nthreads=NT)[:2]
    _check(yg[:, cols], y, ad, what + " (all rows, sampled columns)")


@pytest.mark.parametrize("gemm", ["a4w4", "a8w8"])
def test_256_row_tiles_unaligned_output(mx, orc, gemm):
    """More than 160 tiles of 256 x 256 with N % 8 != 0, where 256 x 224 tiles would take more rounds
    (240 tiles against 276): the 256 x 256 tile kernels with element-wise output stores
    (gemm_tile_fp4<false, 256>, gemm_tile_fp8<false>), on sampled rows and columns."""
    M, N, K = 3072, 5001, 1024
    ops = (_random_mx if gemm == "a4w4" else _random_ptpc)(orc, 901 if gemm == "a4w4" else 902, M, N, K)
    _sampled_check(mx, orc, *ops, "%s 256-row tiles %dx%dx%d" % (gemm, M, N, K), 903, gemm=gemm)


def test_a4w4_prefill_config_sampled(mx, orc):
    cfg = synth.CONFIGS["oproj_prefill_a4w4"]
    qw, sw = _weight_mx("oproj_prefill_a4w4")
    qa, sa = orc.mx_quant_bf16(synth.make_activations(cfg), nthreads=NT)
    _sampled_check(mx, orc, qa, sa, qw, sw, "o_proj prefill 8192x7168x8192", 31)


@pytest.mark.parametrize("M", [1, 16, 128, 512, 2048])
def test_a4w4_msweep_outliers(mx, orc, M):
    cfg = synth.CONFIGS["msweep_outlier_a4w4"]
    qw, sw = _weight_mx("msweep_outlier_a4w4")
    qa, sa = orc.mx_quant_bf16(synth.make_activations(cfg, M), nthreads=NT)
    if M <= 128:
        y, ad, span = orc.gemm_a4w4_at(qa, sa, qw, sw, nthreads=NT)
        _check(_a4w4_gpu(mx, qa, sa, qw, sw), y, ad, "outlier sweep M=%d" % M)
    else:
        _sampled_check(mx, orc, qa, sa, qw, sw, "outlier sweep M=%d" % M, 40 + M)


def test_a4w4_nan_scale_propagates(mx, orc):
    qa, sa, qw, sw = _random_mx(orc, 5, 4, 64, 256)
    sa = sa.copy()
    sw = sw.copy()
    sa[1, 3] = 0xFF
    sw[7, 0] = 0xFF
    y, ad, _ = orc.gemm_a4w4_at(qa, sa, qw, sw)
    _check(_a4w4_gpu(mx, qa, sa, qw, sw), y, ad, "NaN scales")


def test_a4w4_deterministic_and_guarded(mx, orc):
    import torch
    for M, N, K in [(37, 1000, 1024), (100, 1000, 2048), (300, 700, 1024)]:
        qa, sa, qw, sw = _random_mx(orc, 77 + M, M, N, K)
        pad = 4096
        buf = torch.full((M * N + 2 * pad,), -12345.0, dtype=torch.bfloat16, device="cuda")
        y1 = buf[pad:pad + M * N].view(M, N)
        mx.gemm_a4w4(to_dev(qa), to_dev(sa), to_dev(qw), to_dev(sw), y=y1)
        y2 = mx.gemm_a4w4(to_dev(qa), to_dev(sa), to_dev(qw), to_dev(sw))
        torch.cuda.synchronize()
        assert torch.equal(y1.view(torch.int16), y2.view(torch.int16)), "two runs differ"
        sentinel = torch.tensor(-12345.0).to(torch.bfloat16).float().item()
        guard = torch.cat([buf[:pad], buf[pad + M * N:]]).float()
        assert bool((guard == sentinel).all()), "a write landed outside Y"


# --------------------------------------------------------------- A8W8
def _random_ptpc(orc, seed, M, N, K):
    x = synth.f64_to_bf16_bits(synth.normal(seed, M * K)).reshape(M, K)
    w = synth.weight_normal(seed + 1, N, K, 0.01)
    qa, sa = orc.ptpc_quant_bf16(x, nthreads=NT)
    qw, sw = orc.ptpc_quant_f32(w, nthreads=NT)
    return qa, sa, qw, sw


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_a8w8_shapes(mx, orc, M, N, K):
    qa, sa, qw, sw = _random_ptpc(orc, M * 5 + N + K, M, N, K)
    y, ad = orc.gemm_a8w8_at(qa, sa, qw, sw, nthreads=NT)
    _check(_a8w8_gpu(mx, qa, sa, qw, sw), y, ad, "a8w8 %dx%dx%d" % (M, N, K))


@pytest.mark.parametrize("M,N,K", [(16, 40, 1024), (200, 72, 640)])
def test_a8w8_every_code(mx, orc, M, N, K):
    # codes drawn over all 254 finite E4M3 values (subnormals included) on both sides
    rng = np.random.default_rng(M + N)
    qa = rng.integers(0, 256, (M, K), dtype=np.uint8)
    qw = rng.integers(0, 256, (N, K), dtype=np.uint8)
    qa = np.where((qa & 0x7F) == 0x7F, qa ^ 1, qa).astype(np.uint8)
    qw = np.where((qw & 0x7F) == 0x7F, qw ^ 1, qw).astype(np.uint8)
    sa = (rng.random(M) * 2.0 ** -6).astype(np.float32)
    sw = (rng.random(N) * 2.0 ** -6).astype(np.float32)
    y, ad = orc.gemm_a8w8_at(qa, sa, qw, sw)
    _check(_a8w8_gpu(mx, qa, sa, qw, sw), y, ad, "a8w8 every code %dx%dx%d" % (M, N, K))


def test_a8w8_m64_config_full(mx, orc):
    cfg = synth.CONFIGS["ptpc_a8w8_m64"]
    qw, sw = _weight_ptpc("ptpc_a8w8_m64")
    qa, sa = orc.ptpc_quant_bf16(synth.make_activations(cfg))
    y, ad = orc.gemm_a8w8_at(qa, sa, qw, sw, nthreads=NT)
    _check(_a8w8_gpu(mx, qa, sa, qw, sw), y, ad, "PTPC 64x7168x8192")


def test_a8w8_m8192_config_sampled(mx, orc):
    cfg = synth.CONFIGS["ptpc_a8w8_m8192"]
    qw, sw = _weight_ptpc("ptpc_a8w8_m8192")
    qa, sa = orc.ptpc_quant_bf16(synth.make_activations(cfg), nthreads=NT)
    _sampled_check(mx, orc, qa, sa, qw, sw, "PTPC 8192x7168x8192", 51, gemm="a8w8")


# --------------------------------------------------------------- whole layers (HIP quant + HIP GEMM)
def test_linear_a4w4_layer_decode(mx, orc):
    cfg = synth.CONFIGS["oproj_decode_a4w4"]
    qw, sw = _weight_mx("oproj_decode_a4w4")
    x = synth.make_activations(cfg)
    yg = bf16_host(mx.linear_a4w4(bf16_dev(x), to_dev(qw), to_dev(sw)))
    qa, sa = orc.mx_quant_bf16(x)
    y, ad, _ = orc.gemm_a4w4_at(qa, sa, qw, sw, nthreads=NT)
    _check(yg, y, ad, "A4W4 layer 64x7168x8192")


def test_linear_a8w8_layer_decode(mx, orc):
    cfg = synth.CONFIGS["ptpc_a8w8_m64"]
    qw, sw = _weight_ptpc("ptpc_a8w8_m64")
    x = synth.make_activations(cfg)
    yg = bf16_host(mx.linear_a8w8(bf16_dev(x), to_dev(qw), to_dev(sw)))
    qa, sa = orc.ptpc_quant_bf16(x)
    y, ad = orc.gemm_a8w8_at(qa, sa, qw, sw, nthreads=NT)
    _check(yg, y, ad, "A8W8 layer 64x7168x8192")
