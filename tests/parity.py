"""Parity helpers shared by the GPU tests: device transfer and the GEMM acceptance rule.

GEMM acceptance (per element): |y_gpu - y_exact| <= 2^-8 * |y_exact| + 1e-6 * sum_k |a_k * w_k|,
with a, w the dequantized operands and y_exact the oracle's exact value; a NaN
exact value must come back as NaN.  Quantizers are compared bit for bit.
"""
import numpy as np

TOL_REL = 2.0 ** -8
TOL_ABS = 1e-6


def to_dev(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


def bf16_dev(bits):
    import torch
    return to_dev(np.ascontiguousarray(bits, np.uint16).view(np.int16), torch.bfloat16)


def bf16_host(t):
    """BF16 device tensor -> float64 numpy."""
    import torch
    u = t.detach().cpu().view(torch.int16).numpy().view(np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def gemm_within_tolerance(y_gpu, y_exact, absdot):
    """Returns (all_ok, max err/bound ratio, count of violations)."""
    y_gpu = np.asarray(y_gpu, np.float64)
    nan_exact = np.isnan(y_exact)
    if not np.array_equal(np.isnan(y_gpu), nan_exact):
        return False, float("inf"), int((np.isnan(y_gpu) != nan_exact).sum())
    ok = ~nan_exact
    err = np.abs(y_gpu[ok] - y_exact[ok])
    bound = TOL_REL * np.abs(y_exact[ok]) + TOL_ABS * absdot[ok]
    bad = err > bound
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bound > 0, err / bound, np.where(err > 0, np.inf, 0.0))
    return (not bad.any()), float(ratio.max() if ratio.size else 0.0), int(bad.sum())
