"""Pins for the oracle's element/scale decoders and element encoders.

Each pin comes from somewhere other than the oracle's own code: the OCP
format value tables, torch's CPU dtype casts (library routines), or an
independently written threshold rule.  Formats: "Kimi-K3 DSpark O-Proj-only
MXFP4", section "Exact quantization coverage" (E2M1 / E8M0);
"Kimi-K3-DSpark-FP8-PTPC", section "Phase 1 FP8 PTPC Quantization"
(float8_e4m3fn).
"""
import math

import numpy as np
import pytest
import torch


# --------------------------------------------------------------- decoders
def test_e2m1_table_matches_published_grid(orc):
    # the OCP E2M1 value set, sign-magnitude, code 8 is -0
    pos = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    t = orc.e2m1_table()
    assert list(t[:8]) == pos
    assert list(t[8:]) == [-v for v in pos]
    assert math.copysign(1.0, t[8]) == -1.0


def test_e8m0_decode_vs_torch(orc):
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = orc.e8m0_table()
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert np.array_equal(got[:255], ref[:255])
    assert got[0] == 2.0 ** -127 and got[127] == 1.0 and got[254] == 2.0 ** 127


def test_e4m3fn_decode_vs_torch(orc):
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = orc.e4m3fn_table()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert nan.sum() == 2  # 0x7F and 0xFF
    assert np.array_equal(got[~nan], ref[~nan])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9


def test_bf16_decode_vs_torch_all_patterns(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([orc.bf16_value(int(b)) for b in bits])
    r = ref
    assert np.array_equal(np.isnan(got), np.isnan(r))
    ok = ~np.isnan(r)
    assert np.array_equal(got[ok], r[ok])


# --------------------------------------------------------------- E2M1 encode
def _e2m1_by_thresholds(t):
    """Independent rule: the grid midpoints, with the tie going to the even code."""
    if t <= 0.25:
        return 0
    if t < 0.75:
        return 1
    if t <= 1.25:
        return 2
    if t < 1.75:
        return 3
    if t <= 2.5:
        return 4
    if t < 3.5:
        return 5
    if t <= 5.0:
        return 6
    return 7


def _bf16_positive_values_below(limit):
    bits = np.arange(0, 0x7F80, dtype=np.uint32)
    vals = (bits << 16).view(np.float32).astype(np.float64)
    return vals[vals < limit]


def test_e2m1_encode_vs_threshold_rule(orc):
    ts = set(np.arange(0, 10 * 1024 + 1) / 1024.0)  # dense grid incl. every midpoint
    ts.update(_bf16_positive_values_below(16.0)[::7])  # every scaled BF16 magnitude class
    ts.update([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.999, 1e-30, 5e-324])
    for t in sorted(ts):
        assert orc.e2m1_encode(float(t)) == _e2m1_by_thresholds(t), t


def test_e2m1_encode_ties_go_to_even_code(orc):
    # the seven midpoints between adjacent grid values
    assert [orc.e2m1_encode(t) for t in (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)] == [0, 2, 2, 4, 4, 6, 6]
    # saturation: everything above 6 clamps to 6 (code 7)
    assert [orc.e2m1_encode(t) for t in (6.0, 6.5, 7.9, 1e9)] == [7, 7, 7, 7]


# --------------------------------------------------------------- E4M3 encode
def _e4m3_via_oracle_rows(orc, xs):
    """Encode many values with the row quantizer: a leading 448 fixes the row
    scale to exactly 1.0 (448 / 448), so every code is the plain encoding of x."""
    xs = np.asarray(xs, np.float32)
    n = xs.size
    width = 4096
    rows = (n + width - 2) // (width - 1)
    buf = np.zeros((rows, width), np.float32)
    buf[:, 0] = 448.0
    flat = np.zeros(rows * (width - 1), np.float32)
    flat[:n] = xs
    buf[:, 1:] = flat.reshape(rows, width - 1)
    q, s = orc.ptpc_quant_f32(buf)
    assert np.all(s == 1.0)
    return q[:, 1:].reshape(-1)[:n]


def _torch_e4m3(xs):
    return torch.from_numpy(np.asarray(xs, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3fn_encode_vs_torch_strided_float32(orc):
    top = np.frombuffer(np.float32(448.0).tobytes(), np.uint32)[0]
    bits = np.arange(0, top + 1, 97, dtype=np.uint32)
    xs = bits.view(np.float32)
    got = _e4m3_via_oracle_rows(orc, xs)
    assert np.array_equal(got, _torch_e4m3(xs))
    got_neg = _e4m3_via_oracle_rows(orc, -xs[::5])
    assert np.array_equal(got_neg, _torch_e4m3(-xs[::5]))


def test_e4m3fn_encode_vs_torch_around_every_midpoint(orc):
    vals = orc.e4m3fn_table()[:0x7F]
    mids = (vals[:-1] + vals[1:]) / 2.0
    pts = []
    for m in list(mids) + list(vals):
        b = np.frombuffer(np.float32(m).tobytes(), np.uint32)[0].astype(np.int64)
        pts.append(np.arange(max(b - 64, 0), b + 65, dtype=np.int64))
    bits = np.unique(np.concatenate(pts)).astype(np.uint32)
    xs = bits.view(np.float32)
    xs = xs[xs <= 448.0]
    got = _e4m3_via_oracle_rows(orc, xs)
    assert np.array_equal(got, _torch_e4m3(xs))


def test_e4m3fn_encode_saturates_above_448(orc):
    # torch's cast keeps RNE up to the 464 tie and returns NaN beyond; the
    # reading taken here clamps every finite magnitude above 448 to 448.
    for v in (448.0, 449.0, 463.9, 464.0, 500.0, 1e30, float("inf")):
        assert orc.e4m3fn_encode(v) == 0x7E
        assert orc.e4m3fn_encode(-v) == 0xFE
    assert orc.e4m3fn_encode(float("nan")) == 0x7F
    assert orc.e4m3fn_encode(-0.0) == 0x80
