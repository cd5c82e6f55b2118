"""Reference GEMMs: dequantize every operand to fp64, then multiply.

TEST INFRASTRUCTURE (oracle).  Importable only by the tests, the smoke check
and the benchmark's CPU-baseline leg.

Each variant's result has a plain definition -- the product of the
dequantized operands -- and that definition is what is written here, with
NumPy's fp64 matmul as the one library step.  The W4A16 page (section 1) shows
exactly this dequantize-then-multiply form as the naive path the fused kernel
replaces; it is the reference, never the product.

Pinned in tests/test_oracle_pins.py by exact rational brute force on tiny
shapes, one-hot read-back of the dequantized weights, and closed forms.
"""

import numpy as np

from .formats import unpack_int4_along_k, e4m3fn_decode
from .quantize import mxfp4_dequant

INT4_ZERO_POINT = 8     # W4A16 page, section 2: code minus 8, times the scale


def _as_f64(a):
    return np.asarray(a).astype(np.float64)


def dequant_w4(packed, scales):
    """[K/2, N] packed INT4 + [N] fp16 scale -> fp64 [K, N]: (code - 8) * s[n].

    W4A16 page, section 2: unpack the nibble, subtract 8, multiply by the
    column's scale.  The page does this in fp16; the oracle keeps the exact
    value (it needs at most 4 + 11 significant bits).
    """
    codes = unpack_int4_along_k(packed).astype(np.int64)
    s = np.asarray(scales)
    if s.ndim != 1 or s.shape[0] != codes.shape[1]:
        raise ValueError("one scale per output column")
    return (codes - INT4_ZERO_POINT).astype(np.float64) * _as_f64(s)[None, :]


def dequant_w8(w, scales):
    """[K, N] int8 + [N] fp16 scale -> fp64 [K, N]: w * s[n].

    W8A16 page, Step 1: Y = X (W_int8 * S) with one scale per column.
    """
    w = np.asarray(w)
    if w.dtype != np.int8 or w.ndim != 2:
        raise ValueError("W8 weights must be a 2-D int8 array")
    s = np.asarray(scales)
    if s.ndim != 1 or s.shape[0] != w.shape[1]:
        raise ValueError("one scale per output column")
    return w.astype(np.float64) * _as_f64(s)[None, :]


def _product_and_bound(a, b):
    """Return (a @ b, |a| @ |b|) in fp64."""
    return a @ b, np.abs(a) @ np.abs(b)


def gemm_w4a16(x, packed, scales):
    """Y = X @ W_deq for X fp16 [M, K] and packed INT4 [K/2, N].

    Returns (Y fp64 [M, N], bound fp64 [M, N]) where bound = |X| @ |W_deq|
    feeds the error tolerance.  The device result is fp16.
    """
    return _product_and_bound(_as_f64(x), dequant_w4(packed, scales))


def gemm_w8a16(x, w, scales):
    """Y = X @ (W_int8 * S) for X fp16 [M, K], W int8 [K, N] (W8A16 page, Step 1)."""
    return _product_and_bound(_as_f64(x), dequant_w8(w, scales))


def gemm_mxfp4(a_codes, a_e8m0, w_codes, w_e8m0):
    """C = A_deq @ W_deq^T for MXFP4 A [M, K] and W [N, K].

    MXFP4 page, section 2: A is M x K, W is N x K, and C is M x N; eq. (1)
    sums per-block scaled dot products, which equals the product of the
    dequantized operands.  The device result is bf16.
    """
    a = mxfp4_dequant(a_codes, a_e8m0)
    w = mxfp4_dequant(w_codes, w_e8m0)
    return _product_and_bound(a, w.T)


def gemm_fp8(a_codes, b_codes, scale_a, scale_b):
    """C = (q_a @ q_b) * scale_a * scale_b for e4m3fn A [M, K] and B [K, N].

    FP8 page: the dot product runs on e4m3fn codes with an fp32 accumulator and
    the per-tensor scales multiply the accumulator; the output is bf16.  The
    bound uses the dequantized operands |q_a * s_a| @ |q_b * s_b|.
    """
    qa = e4m3fn_decode(a_codes)
    qb = e4m3fn_decode(b_codes)
    sa = float(np.float32(scale_a))
    sb = float(np.float32(scale_b))
    c = (qa @ qb) * sa * sb
    bound = (np.abs(qa) * sa) @ (np.abs(qb) * sb)
    return c, bound


def tolerance(bound):
    """Allowed |Y - Y_ref|: 1e-2 * (|X| @ |W_deq|) + 1e-3, elementwise."""
    return 1e-2 * np.asarray(bound, dtype=np.float64) + 1e-3


def within_tolerance(y, y_ref, bound):
    """Boolean array: does each output satisfy the error bound?"""
    y = np.asarray(y, dtype=np.float64)
    return np.abs(y - y_ref) <= tolerance(bound)
