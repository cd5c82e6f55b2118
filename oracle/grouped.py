"""Group-wise scales and asymmetric zero points for the weight-only GEMMs.

TEST INFRASTRUCTURE (oracle).  Importable only by the tests, the smoke check
and the benchmark's CPU-baseline leg.

Sources:
* W4A16 page, section 1: the naive path dequantizes as
  (w_int4 - zero_point) * scale before the matmul.
* W8A16 page, extensions: group-wise quantization lets several columns share
  one scale; introducing a zero point turns the symmetric scheme asymmetric.
  The same page names GPTQ/AWQ (intro), whose groups run along K.

Reading: the scale and the zero point are indexed by a group along K and a
group along N, s[k // group_k, n // group_n] and z[k // group_k, n // group_n];
group_k = K with group_n = 1 is the per-column scheme of the W4A16 and W8A16
pages, group_n > 1 is the page's column sharing and group_k < K the GPTQ/AWQ
grouping.  W4: codes 0..15 and zero points 0..15 (default 8, the W4A16 page's
symmetric zero point).  W8: int8 weights and int8 zero points (default 0).
The dequantized weight is the exact value (c - z) * s, as for the per-column
oracle; the result is X @ W_deq in fp64.

Pinned in tests/test_oracle_grouped.py: reduction to the per-column routines,
exact rational brute force on tiny shapes, the single-group zero-point closed
form, and group locality.
"""

import numpy as np

from .formats import unpack_int4_along_k
from .gemm import INT4_ZERO_POINT


def _cdiv(a, b):
    return -(-a // b)


def expand_groups(table, k, n, group_k, group_n):
    """[ceil(K/group_k), ceil(N/group_n)] -> [K, N]: entry (k, n) of the result
    is table[k // group_k, n // group_n]."""
    t = np.asarray(table)
    if group_k < 1 or group_n < 1:
        raise ValueError("group sizes must be positive")
    if t.shape != (_cdiv(k, group_k), _cdiv(n, group_n)):
        raise ValueError(f"group table must be {(_cdiv(k, group_k), _cdiv(n, group_n))}, got {t.shape}")
    return t[np.arange(k) // group_k][:, np.arange(n) // group_n]


def dequant_w4_grouped(packed, scales, zeros, group_k, group_n=1):
    """[K/2, N] packed INT4 -> fp64 [K, N]: (code - z) * s per (K group, N group).

    zeros=None means the symmetric zero point 8 everywhere."""
    codes = unpack_int4_along_k(packed).astype(np.int64)
    k, n = codes.shape
    s = expand_groups(scales, k, n, group_k, group_n).astype(np.float64)
    if zeros is None:
        z = np.full((k, n), INT4_ZERO_POINT, np.int64)
    else:
        zt = np.asarray(zeros)
        if zt.dtype != np.uint8 or zt.size and int(zt.max()) > 15:
            raise ValueError("W4 zero points are uint8 values 0..15")
        z = expand_groups(zt, k, n, group_k, group_n).astype(np.int64)
    return (codes - z).astype(np.float64) * s


def dequant_w8_grouped(w, scales, zeros, group_k, group_n=1):
    """[K, N] int8 -> fp64 [K, N]: (w - z) * s per (K group, N group).

    zeros=None means zero point 0 (the W8A16 page's symmetric scheme)."""
    w = np.asarray(w)
    if w.dtype != np.int8 or w.ndim != 2:
        raise ValueError("W8 weights must be a 2-D int8 array")
    k, n = w.shape
    s = expand_groups(scales, k, n, group_k, group_n).astype(np.float64)
    if zeros is None:
        z = np.zeros((k, n), np.int64)
    else:
        zt = np.asarray(zeros)
        if zt.dtype != np.int8:
            raise ValueError("W8 zero points are int8")
        z = expand_groups(zt, k, n, group_k, group_n).astype(np.int64)
    return (w.astype(np.int64) - z).astype(np.float64) * s


def gemm_w4a16_grouped(x, packed, scales, zeros, group_k, group_n=1):
    """(Y = X @ W_deq, bound = |X| @ |W_deq|) in fp64 for grouped INT4 weights."""
    wd = dequant_w4_grouped(packed, scales, zeros, group_k, group_n)
    xd = np.asarray(x).astype(np.float64)
    return xd @ wd, np.abs(xd) @ np.abs(wd)


def gemm_w8a16_grouped(x, w, scales, zeros, group_k, group_n=1):
    """(Y = X @ W_deq, bound = |X| @ |W_deq|) in fp64 for grouped INT8 weights."""
    wd = dequant_w8_grouped(w, scales, zeros, group_k, group_n)
    xd = np.asarray(x).astype(np.float64)
    return xd @ wd, np.abs(xd) @ np.abs(wd)
