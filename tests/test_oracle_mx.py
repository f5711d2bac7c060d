"""Pins for the oracle's MXFP4 quantizer (E2M1 codes + one E8M0 scale per 32 K-values).

Format: "Kimi-K3 DSpark O-Proj-only MXFP4", section "Exact quantization coverage";
standard named "OCP MXFP4" by "Kimi-K3-Quark-MXFP4-AttnFP8", section "Model
Quantization".  Pins: hand-worked golden block, the checkpoint-size row the page
prints, an independent shared-exponent rule read off the BF16 exponent field,
and invariants (power-of-two scaling, negation, saturation, error bound).
"""
import numpy as np
import pytest

from block_scaled_precision_act_amd import synth
from golden_io import read


def _bf16(vals):
    return synth.f64_to_bf16_bits(np.asarray(vals, np.float64))


def _unpack(q):
    codes = np.empty(q.shape[:-1] + (q.shape[-1] * 2,), np.uint8)
    codes[..., 0::2] = q & 15
    codes[..., 1::2] = q >> 4
    return codes


# --------------------------------------------------------------- golden
def test_golden_block(orc):
    g = read("mx_block_1x32.txt")
    v = np.array([float(t) for t in g["input"]])
    codes, scale = orc.mx_block(v)
    assert scale == int(g["scale"][0], 16)
    assert [int(c) for c in codes] == [int(c, 16) for c in g["codes"]]
    # row quantizer: same block through the BF16 entry, packed low nibble first
    q, s = orc.mx_quant_bf16(_bf16(v)[None, :])
    assert list(q[0]) == [int(b, 16) for b in g["packed"]]
    assert s[0, 0] == int(g["scale"][0], 16)
    codes2, scale2 = orc.mx_block(v * 2.0 ** -10)
    assert scale2 == int(g["scale_times_2^-10"][0], 16)
    assert np.array_equal(codes2, codes)


def test_special_blocks(orc):
    z = np.zeros(32)
    c, s = orc.mx_block(z)
    assert s == 0 and not c.any()
    c, s = orc.mx_block(-z)
    assert s == 0 and np.all(c == 8)  # sign of -0 kept
    c, s = orc.mx_block(np.full(32, 2.0 ** -130))
    assert s == 0 and not c.any()  # 2^-130 / 2^-127 = 1/8 rounds to 0
    v = np.zeros(32)
    v[0] = 2.0 ** -126
    c, s = orc.mx_block(v)
    assert s == 0 and c[0] == 4  # 2^-126 / 2^-127 = 2 -> code 4
    for bad in (np.nan, np.inf, -np.inf):
        v = np.ones(32)
        v[5] = bad
        c, s = orc.mx_block(v)
        assert s == 0xFF and not c.any()


# --------------------------------------------------------------- page pin
def test_checkpoint_size_delta_matches_page(orc):
    g = read("checkpoint_sizes.txt")
    L, N, K = int(g["layers"][0]), int(g["out_features"][0]), int(g["in_features"][0])
    row = synth.weight_normal(1, 1, K, 0.02)
    q, s = orc.mx_quant_f32(row)
    assert s.shape[1] == int(g["mx_scale_cols"][0])  # (7168, 256) scale shape on the page
    q8, s8 = orc.ptpc_quant_f32(row)
    mx_bytes = N * (q.nbytes + s.nbytes)
    fp8_bytes = N * (q8.nbytes + s8.nbytes)
    delta_gib = L * (fp8_bytes - mx_bytes) / 2.0 ** 30
    page_delta = float(g["gib_fp8"][0]) - float(g["gib_mxfp4"][0])
    assert round(delta_gib, 2) == round(page_delta, 2)
    assert mx_bytes * 8 / (N * K) == 4.25  # 4 bits per element + one byte per 32


# --------------------------------------------------------------- independent rules
def _blocks_bank():
    rng_blocks = [
        synth.f64_to_bf16_bits(synth.normal(11, 32 * 512)),
        synth.f64_to_bf16_bits(synth.student_t3(12, 32 * 512) * 50.0),
        synth.f64_to_bf16_bits(synth.normal(13, 32 * 256) * 2.0 ** -125),  # tiny / subnormal
        synth.f64_to_bf16_bits(synth.normal(14, 32 * 256) * 2.0 ** 120),   # huge
    ]
    b = np.concatenate(rng_blocks).reshape(-1, 32)
    # sprinkle exact zeros and exact grid ties
    b[::7, 3] = 0
    b[::5, 9] = _bf16([1.75])[0]
    return b


def test_shared_exponent_from_exponent_field(orc):
    bits = _blocks_bank()
    q, s = orc.mx_quant_bf16(bits.reshape(1, -1))
    efield = ((bits >> 7) & 0xFF).astype(np.int64)  # BF16 biased exponent field
    expect = np.maximum(efield.max(axis=1) - 2, 0)
    assert np.array_equal(s[0].astype(np.int64), expect)


def _threshold_code(t):
    edges_incl = [(0.25, True), (0.75, False), (1.25, True), (1.75, False), (2.5, True), (3.5, False), (5.0, True)]
    code = np.zeros(t.shape, np.uint8)
    for edge, tie_stays_below in edges_incl:
        code += (t > edge) if tie_stays_below else (t >= edge)
    return code


def test_element_codes_threshold_rule(orc):
    bits = _blocks_bank()
    q, s = orc.mx_quant_bf16(bits.reshape(1, -1))
    codes = _unpack(q).reshape(-1, 32)
    x = synth.bf16_bits_to_f32(bits).astype(np.float64)
    e = s[0].astype(np.int64) - 127
    t = np.abs(x) * np.exp2(-e)[:, None]
    expect = _threshold_code(t) | (np.signbit(x).astype(np.uint8) << 3)
    assert np.array_equal(codes, expect)


# --------------------------------------------------------------- invariants
def test_power_of_two_scaling_invariant(orc):
    x = synth.normal(21, 64 * 256).reshape(64, 256)
    q0, s0 = orc.mx_quant_f32(x.astype(np.float32))
    for j in (-40, -3, 1, 17, 60):
        q1, s1 = orc.mx_quant_f32((x * 2.0 ** j).astype(np.float32))
        assert np.array_equal(q1, q0)
        assert np.array_equal(s1.astype(int), s0.astype(int) + j)


def test_negation_flips_sign_nibbles(orc):
    x = synth.normal(22, 16 * 512).reshape(16, 512).astype(np.float32)
    q0, s0 = orc.mx_quant_f32(x)
    q1, s1 = orc.mx_quant_f32(-x)
    assert np.array_equal(s0, s1)
    assert np.array_equal(q1, q0 ^ 0x88)


def test_block_max_lands_on_top_of_grid_and_error_bound(orc):
    x = synth.normal(23, 256 * 128).reshape(256, 128)
    q, s = orc.mx_quant_f32(x.astype(np.float32))
    xf = x.astype(np.float32).astype(np.float64)
    deq = orc.dequant_mx(q, s)
    codes = _unpack(q)
    blocks = np.abs(xf).reshape(256, 4, 32)
    argmax = blocks.argmax(axis=2)
    top = np.take_along_axis(codes.reshape(256, 4, 32), argmax[..., None], axis=2)[..., 0] & 7
    assert np.all((top == 6) | (top == 7))  # max/2^e in [4, 8) -> 4 or 6
    scale = np.repeat(np.exp2(s.astype(np.float64) - 127), 32, axis=1)
    t = np.abs(xf) / scale
    # within the grid's half step (0.25 below 2, 0.5 below 4, 1 below 6) or clamped to 6
    half = np.where(t < 2, 0.25, np.where(t < 4, 0.5, 1.0))
    err = np.abs(np.abs(deq) - np.abs(xf)) / scale
    ok = (err <= half) | ((t > 6) & (np.abs(deq) / scale == 6))
    assert ok.all()


def test_bf16_and_f32_entries_agree(orc):
    bits = synth.act_normal(24, 8, 1024)
    qa, sa = orc.mx_quant_bf16(bits)
    qb, sb = orc.mx_quant_f32(synth.bf16_bits_to_f32(bits))
    assert np.array_equal(qa, qb) and np.array_equal(sa, sb)


def test_bad_arguments_rejected(orc):
    with pytest.raises(ValueError):
        orc.mx_quant_f32(np.zeros((2, 33), np.float32))
