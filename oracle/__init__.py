"""CPU parity oracle for the block-scaled linear layer (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: the test-suite, the package smoke check and the
CPU-baseline leg of the benchmark are the only users.  The product library
never imports this package and shares no code with it.

The arithmetic lives in ``oracle.c`` (plain C11, see ``oracle.h`` for the
definitions and the readings of the pages it follows).  This module only
marshals numpy arrays in and out and builds the C file with gcc when the
shared object is missing or older than its source.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
(exhaustive decoder tables, library casts, brute force, hand-worked golden
examples and invariants); none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_HDR = os.path.join(_HERE, "oracle.h")
_LIB = os.path.join(_HERE, "liboracle.so")

OK, EARG, EINEXACT = 0, -1, -2


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with plain gcc (no fast-math)."""
    stale = (not os.path.exists(_LIB)
             or os.path.getmtime(_LIB) < max(os.path.getmtime(_SRC), os.path.getmtime(_HDR)))
    if force or stale:
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
             "-Wall", "-Wextra", "-o", tmp, _SRC, "-lpthread", "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        c_u8p = ctypes.POINTER(ctypes.c_uint8)
        i64, i32 = ctypes.c_int64, ctypes.c_int
        vp = ctypes.c_void_p
        for name in ("orc_e2m1_value", "orc_e8m0_value", "orc_e4m3fn_value"):
            getattr(lib, name).argtypes = [ctypes.c_uint]
            getattr(lib, name).restype = ctypes.c_double
        lib.orc_bf16_value.argtypes = [ctypes.c_uint16]
        lib.orc_bf16_value.restype = ctypes.c_double
        lib.orc_e2m1_encode.argtypes = [ctypes.c_double]
        lib.orc_e2m1_encode.restype = ctypes.c_uint
        lib.orc_e4m3fn_encode.argtypes = [ctypes.c_double]
        lib.orc_e4m3fn_encode.restype = ctypes.c_uint
        lib.orc_mx_block.argtypes = [vp, vp, c_u8p]
        lib.orc_mx_block.restype = None
        for name in ("orc_mx_quant_bf16", "orc_mx_quant_f32", "orc_ptpc_quant_bf16", "orc_ptpc_quant_f32"):
            getattr(lib, name).argtypes = [vp, i64, i64, vp, vp, i32]
            getattr(lib, name).restype = i32
        lib.orc_gemm_a4w4_at.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp, i64, vp, i64, vp, vp,
                                         ctypes.POINTER(ctypes.c_int), i32]
        lib.orc_gemm_a4w4_at.restype = i32
        lib.orc_gemm_a8w8_at.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp, i64, vp, i64, vp, vp, i32]
        lib.orc_gemm_a8w8_at.restype = i32
        _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data) if a.size else ctypes.c_void_p(0)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------- decoders
def e2m1_value(code: int) -> float:
    return _load().orc_e2m1_value(code)


def e8m0_value(code: int) -> float:
    return _load().orc_e8m0_value(code)


def e4m3fn_value(code: int) -> float:
    return _load().orc_e4m3fn_value(code)


def bf16_value(bits: int) -> float:
    return _load().orc_bf16_value(bits)


def e2m1_encode(t: float) -> int:
    return _load().orc_e2m1_encode(t)


def e4m3fn_encode(r: float) -> int:
    return _load().orc_e4m3fn_encode(r)


def e2m1_table() -> np.ndarray:
    return np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)


def e4m3fn_table() -> np.ndarray:
    return np.array([e4m3fn_value(c) for c in range(256)], dtype=np.float64)


def e8m0_table() -> np.ndarray:
    return np.array([e8m0_value(c) for c in range(256)], dtype=np.float64)


# ---------------------------------------------------------------- MX
def mx_block(v) -> tuple[np.ndarray, int]:
    """One 32-value block -> (32 unpacked E2M1 codes, E8M0 scale byte)."""
    v = _c(v, np.float64)
    assert v.shape == (32,)
    codes = np.zeros(32, np.uint8)
    sc = ctypes.c_uint8(0)
    _load().orc_mx_block(_ptr(v), _ptr(codes), ctypes.byref(sc))
    return codes, int(sc.value)


def _mx(fn, x, dtype, nthreads):
    x = _c(x, dtype)
    if x.ndim != 2:
        raise ValueError("expected a 2-D array")
    rows, K = x.shape
    q = np.zeros((rows, K // 2), np.uint8)
    s = np.zeros((rows, K // 32), np.uint8)
    rc = fn(_ptr(x), rows, K, _ptr(q), _ptr(s), nthreads or default_threads())
    if rc != OK:
        raise ValueError("oracle MX quantizer rejected the arguments (rc=%d)" % rc)
    return q, s


def mx_quant_bf16(x_bits, nthreads: int = 0):
    """BF16 bit patterns [rows, K] -> (codes [rows, K/2], scales [rows, K/32])."""
    return _mx(_load().orc_mx_quant_bf16, x_bits, np.uint16, nthreads)


def mx_quant_f32(x, nthreads: int = 0):
    """FP32 [rows, K] -> (codes [rows, K/2], scales [rows, K/32])."""
    return _mx(_load().orc_mx_quant_f32, x, np.float32, nthreads)


# ---------------------------------------------------------------- PTPC
def _ptpc(fn, x, dtype, nthreads):
    x = _c(x, dtype)
    if x.ndim != 2:
        raise ValueError("expected a 2-D array")
    rows, K = x.shape
    q = np.zeros((rows, K), np.uint8)
    s = np.zeros((rows,), np.float32)
    rc = fn(_ptr(x), rows, K, _ptr(q), _ptr(s), nthreads or default_threads())
    if rc != OK:
        raise ValueError("oracle PTPC quantizer rejected the arguments (rc=%d)" % rc)
    return q, s


def ptpc_quant_bf16(x_bits, nthreads: int = 0):
    """BF16 bit patterns [rows, K] -> (E4M3fn codes [rows, K], FP32 scales [rows])."""
    return _ptpc(_load().orc_ptpc_quant_bf16, x_bits, np.uint16, nthreads)


def ptpc_quant_f32(x, nthreads: int = 0):
    """FP32 [rows, K] -> (E4M3fn codes [rows, K], FP32 scales [rows])."""
    return _ptpc(_load().orc_ptpc_quant_f32, x, np.float32, nthreads)


# ---------------------------------------------------------------- GEMMs
def _grid(M, N, rows, cols):
    rows = np.arange(M, dtype=np.int64) if rows is None else _c(rows, np.int64)
    cols = np.arange(N, dtype=np.int64) if cols is None else _c(cols, np.int64)
    return rows, cols


def gemm_a4w4_at(qa, sa, qw, sw, rows=None, cols=None, nthreads: int = 0, allow_inexact=False):
    """Exact Y = dequant(A) . dequant(W)^T on the grid rows x cols.

    Returns (y [len(rows), len(cols)] float64, absdot (same shape), max_span).
    Raises if the FP64 exactness condition fails, unless allow_inexact."""
    qa, sa, qw, sw = (_c(a, np.uint8) for a in (qa, sa, qw, sw))
    M, K = qa.shape[0], qa.shape[1] * 2
    N = qw.shape[0]
    assert qw.shape == (N, K // 2) and sa.shape == (M, K // 32) and sw.shape == (N, K // 32)
    rows, cols = _grid(M, N, rows, cols)
    y = np.zeros((rows.size, cols.size), np.float64)
    ad = np.zeros_like(y)
    span = ctypes.c_int(0)
    rc = _load().orc_gemm_a4w4_at(_ptr(qa), _ptr(sa), _ptr(qw), _ptr(sw), M, N, K,
                                  _ptr(rows), rows.size, _ptr(cols), cols.size,
                                  _ptr(y), _ptr(ad), ctypes.byref(span), nthreads or default_threads())
    if rc == EINEXACT and not allow_inexact:
        raise ArithmeticError("A4W4 oracle: FP64 exactness condition failed (span %d)" % span.value)
    if rc not in (OK, EINEXACT):
        raise ValueError("oracle A4W4 GEMM rejected the arguments (rc=%d)" % rc)
    return y, ad, int(span.value)


def gemm_a8w8_at(qa, sa, qw, sw, rows=None, cols=None, nthreads: int = 0):
    """Exact Y = sA.sW.(E4M3(A) . E4M3(W)^T) on the grid rows x cols -> (y, absdot)."""
    qa, qw = _c(qa, np.uint8), _c(qw, np.uint8)
    sa, sw = _c(sa, np.float32), _c(sw, np.float32)
    M, K = qa.shape
    N = qw.shape[0]
    assert qw.shape == (N, K) and sa.shape == (M,) and sw.shape == (N,)
    rows, cols = _grid(M, N, rows, cols)
    y = np.zeros((rows.size, cols.size), np.float64)
    ad = np.zeros_like(y)
    rc = _load().orc_gemm_a8w8_at(_ptr(qa), _ptr(sa), _ptr(qw), _ptr(sw), M, N, K,
                                  _ptr(rows), rows.size, _ptr(cols), cols.size,
                                  _ptr(y), _ptr(ad), nthreads or default_threads())
    if rc != OK:
        raise ValueError("oracle A8W8 GEMM rejected the arguments (rc=%d)" % rc)
    return y, ad


# ---------------------------------------------------------------- dequantizers (for pins)
def dequant_mx(q, s) -> np.ndarray:
    """Codes [rows, K/2] + scales [rows, K/32] -> FP64 [rows, K] via the decoders."""
    q = _c(q, np.uint8)
    s = _c(s, np.uint8)
    rows, K = q.shape[0], q.shape[1] * 2
    codes = np.empty((rows, K), np.uint8)
    codes[:, 0::2] = q & 15
    codes[:, 1::2] = q >> 4
    vals = e2m1_table()[codes]
    return vals * np.repeat(e8m0_table()[s], 32, axis=1)


def dequant_ptpc(q, s) -> np.ndarray:
    """E4M3fn codes [rows, K] + FP32 scales [rows] -> FP64 [rows, K]."""
    q = _c(q, np.uint8)
    return e4m3fn_table()[q] * _c(s, np.float32).astype(np.float64)[:, None]
