"""Parity helpers shared by the GPU tests: device transfer and the GEMM acceptance rule.

GEMM acceptance (per element), with a, w the dequantized operands, y the oracle's exact
value and b = 2^-8 * |y| + 1e-6 * sum_k |a_k * w_k| the error bound:
  * a finite GPU value g is accepted when |g - y| <= b + 2^-134;
  * +inf is accepted when y + b reaches BF16's overflow threshold (2 - 2^-8) * 2^127, the
    smallest real that BF16 round-to-nearest-even turns into +inf; -inf symmetrically;
  * a NaN exact value must come back as NaN, and a NaN GPU value needs a NaN exact value.
The 2^-134 term is half the spacing of BF16's subnormals (2^-133): an exact value in the
subnormal range, or below it, has a correctly rounded BF16 result that is up to that far
away (0 below 2^-134), which the relative term cannot cover there.  Everywhere else it is
far below the bound.  The two infinity clauses accept the correctly rounded BF16 result of
an exact value beyond BF16's finite range (and of one that FP32 accumulation error may
push past the threshold).  Quantizers are compared bit for bit.
"""
import numpy as np

TOL_REL = 2.0 ** -8
TOL_ABS = 1e-6
BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127          # largest finite BF16
BF16_OVERFLOW = (2.0 - 2.0 ** -8) * 2.0 ** 127     # RNE rounds |x| >= this to infinity
BF16_HALF_SUBNORMAL = 2.0 ** -134                  # half the spacing of BF16 subnormals


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


def gemm_accepts(y_gpu, y_exact, absdot):
    """Element-wise acceptance mask of the rule above, and the err/bound ratio per element
    (0 for an accepted infinity or NaN, inf for a rejected non-finite value)."""
    g = np.asarray(y_gpu, np.float64)
    y = np.asarray(y_exact, np.float64)
    ad = np.asarray(absdot, np.float64)
    nan_y, nan_g = np.isnan(y), np.isnan(g)
    b = TOL_REL * np.abs(np.where(nan_y, 0.0, y)) + TOL_ABS * np.where(np.isnan(ad), 0.0, ad)
    fin = np.isfinite(g) & ~nan_y
    with np.errstate(invalid="ignore", over="ignore"):
        err = np.where(fin, np.abs(g - np.where(nan_y, 0.0, y)), 0.0)
        lim = b + BF16_HALF_SUBNORMAL
        ok_fin = fin & (err <= lim)
        ok_pinf = (g == np.inf) & ~nan_y & (y + b >= BF16_OVERFLOW)
        ok_ninf = (g == -np.inf) & ~nan_y & (y - b <= -BF16_OVERFLOW)
    ok = np.where(nan_y, nan_g, ok_fin | ok_pinf | ok_ninf)
    ratio = np.where(fin, err / lim, np.where(ok, 0.0, np.inf))
    return ok, ratio


def gemm_within_tolerance(y_gpu, y_exact, absdot):
    """Returns (all_ok, max err/bound ratio, count of violations)."""
    ok, ratio = gemm_accepts(y_gpu, y_exact, absdot)
    return bool(ok.all()), float(ratio.max() if ratio.size else 0.0), int((~ok).sum())
