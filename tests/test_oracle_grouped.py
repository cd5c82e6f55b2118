"""Pins of the grouped (group-wise scale, zero point) weight-only oracle.

The oracle restates the W4A16 page's section 1 dequant form (w - zero_point)
* scale and the W8A16 page's extensions (column-shared scales, zero points);
each pin below checks it against something other than itself.
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle
import qgemm_workloads as wl


def test_expand_groups_indexing():
    t = np.arange(6).reshape(2, 3)
    e = oracle.expand_groups(t, 5, 7, 3, 3)       # K groups {0,1,2},{3,4}; N groups {0..2},{3..5},{6}
    assert e.shape == (5, 7)
    assert e[0, 0] == 0 and e[2, 2] == 0 and e[3, 0] == 3 and e[4, 6] == 5 and e[1, 5] == 1
    with pytest.raises(ValueError):
        oracle.expand_groups(t, 5, 7, 2, 3)        # wrong table shape


@pytest.mark.parametrize("zeros", [None, "eight"])
def test_w4_single_group_per_column_is_the_w4a16_oracle(zeros):
    """group_k = K, group_n = 1, zero point 8: exactly the per-column W4A16 oracle."""
    m, k, n = 5, 96, 24
    x, packed, s = wl.w4a16(m, k, n, seed=3)
    z = None if zeros is None else np.full((1, n), 8, np.uint8)
    y, b = oracle.gemm_w4a16_grouped(x, packed, s[None, :], z, k, 1)
    y0, b0 = oracle.gemm_w4a16(x, packed, s)
    assert np.array_equal(y, y0) and np.array_equal(b, b0)


@pytest.mark.parametrize("zeros", [None, "zero"])
def test_w8_single_group_per_column_is_the_w8a16_oracle(zeros):
    """group_k = K, group_n = 1, zero point 0 (or none given): exactly the
    per-column W8A16 oracle."""
    m, k, n = 4, 80, 20
    x, w, s = wl.w8a16(m, k, n, seed=4)
    z = None if zeros is None else np.zeros((1, n), np.int8)
    y, b = oracle.gemm_w8a16_grouped(x, w, s[None, :], z, k, 1)
    y0, b0 = oracle.gemm_w8a16(x, w, s)
    assert np.array_equal(y, y0) and np.array_equal(b, b0)


def _brute(x, codes, scales, zeros, gk, gn):
    """Exact rational sum, group indices taken per element in the loop."""
    m, k = x.shape
    n = codes.shape[1]
    out = np.empty((m, n), dtype=object)
    for i in range(m):
        for j in range(n):
            acc = Fraction(0)
            for kk in range(k):
                s = Fraction(float(scales[kk // gk][j // gn]))
                z = int(zeros[kk // gk][j // gn])
                acc += Fraction(float(x[i, kk])) * (int(codes[kk, j]) - z) * s
            out[i, j] = acc
    return out


@pytest.mark.parametrize("gk,gn", [(8, 1), (12, 4), (40, 7), (5, 2)])
def test_w4_grouped_matches_exact_rational_sum(gk, gn):
    m, k, n = 3, 40, 9
    x, packed, s, z = wl.w4a16_grouped(m, k, n, gk, gn, seed=gk * 10 + gn)
    y, bound = oracle.gemm_w4a16_grouped(x, packed, s, z, gk, gn)
    codes = oracle.unpack_int4_along_k(packed)
    exact = _brute(x, codes, s, z, gk, gn)
    err = np.abs(y - exact.astype(np.float64))
    assert (err <= 1e-12 * (bound + 1)).all()


@pytest.mark.parametrize("gk,gn", [(16, 1), (7, 3)])
def test_w8_grouped_matches_exact_rational_sum(gk, gn):
    m, k, n = 2, 35, 8
    x, w, s, z = wl.w8a16_grouped(m, k, n, gk, gn, seed=gk + gn)
    y, bound = oracle.gemm_w8a16_grouped(x, w, s, z, gk, gn)
    exact = _brute(x, w, s, z, gk, gn)
    err = np.abs(y - exact.astype(np.float64))
    assert (err <= 1e-12 * (bound + 1)).all()


def test_single_group_zero_point_closed_form():
    """One group for the whole matrix: Y = s * (X @ W - z * rowsum(X))."""
    m, k, n = 6, 64, 10
    x, w, _, _ = wl.w8a16_grouped(m, k, n, k, n, seed=9)
    s = np.array([[0.0078125]], np.float16)
    z = np.array([[-5]], np.int8)
    y, _ = oracle.gemm_w8a16_grouped(x, w, s, z, k, n)
    xd = x.astype(np.float64)
    ref = 0.0078125 * (xd @ w.astype(np.float64) - (-5) * xd.sum(axis=1)[:, None])
    assert np.allclose(y, ref, rtol=1e-13, atol=1e-12)


def test_group_locality():
    """Changing the scale or zero point of group (kg, ng) changes only the
    columns of ng, by exactly X[:, K rows of kg] @ delta."""
    m, k, n, gk, gn = 4, 64, 12, 16, 4
    x, packed, s, z = wl.w4a16_grouped(m, k, n, gk, gn, seed=2)
    y0, _ = oracle.gemm_w4a16_grouped(x, packed, s, z, gk, gn)
    s2, z2 = s.copy(), z.copy()
    s2[1, 2] = np.float16(0.5)
    z2[1, 2] = (int(z[1, 2]) + 3) % 16
    y1, _ = oracle.gemm_w4a16_grouped(x, packed, s2, z2, gk, gn)
    changed = np.abs(y1 - y0) > 0
    cols = np.arange(n) // gn == 2
    assert not changed[:, ~cols].any()
    codes = oracle.unpack_int4_along_k(packed).astype(np.float64)
    rows = slice(gk, 2 * gk)
    d_new = (codes[rows][:, cols] - float(z2[1, 2])) * float(s2[1, 2])
    d_old = (codes[rows][:, cols] - float(z[1, 2])) * float(s[1, 2])
    expect = x.astype(np.float64)[:, rows] @ (d_new - d_old)
    assert np.allclose((y1 - y0)[:, cols], expect, rtol=1e-12, atol=1e-12)


def test_grouped_rejects_bad_zero_points():
    x, packed, s, _ = wl.w4a16_grouped(1, 32, 4, 16, 1, seed=1)
    with pytest.raises(ValueError):
        oracle.gemm_w4a16_grouped(x, packed, s, np.full(s.shape, 16, np.uint8), 16, 1)
    x, w, s, _ = wl.w8a16_grouped(1, 32, 4, 16, 1, seed=1)
    with pytest.raises(ValueError):
        oracle.gemm_w8a16_grouped(x, w, s, np.zeros(s.shape, np.uint8), 16, 1)
