"""Pins of the NVFP4-style weight oracle (two-level block scaling)."""

from fractions import Fraction

import numpy as np
import pytest

import oracle
import qgemm_workloads as wl


def _e2m1_exact(c):
    """E2M1 value from its bit fields: sign, 2 exponent bits (bias 1), 1 mantissa bit."""
    s, e, m = (c >> 3) & 1, (c >> 1) & 3, c & 1
    v = Fraction(m, 2) if e == 0 else Fraction(2) ** (e - 1) * (1 + Fraction(m, 2))
    return -v if s else v


def _e4m3_exact(c):
    """e4m3fn value from its bit fields: bias 7, 3 mantissa bits, subnormals at 0."""
    s, e, m = (c >> 7) & 1, (c >> 3) & 15, c & 7
    v = Fraction(m, 8) * Fraction(2) ** -6 if e == 0 else Fraction(2) ** (e - 7) * (1 + Fraction(m, 8))
    return -v if s else v


def test_matches_exact_rational_sum():
    m, k, n = 3, 64, 5
    x, codes, scales, g = wl.nvfp4_weight(m, k, n, seed=4)
    y, bound = oracle.gemm_nvfp4(x, codes, scales, g)
    gq = Fraction(float(g))
    for i in range(m):
        for j in range(n):
            acc = Fraction(0)
            for kk in range(k):
                byte = int(codes[j, kk // 2])
                c = (byte >> 4) if kk % 2 else (byte & 15)
                acc += Fraction(float(x[i, kk])) * _e2m1_exact(c) * _e4m3_exact(int(scales[j, kk // 16])) * gq
            assert abs(y[i, j] - float(acc)) <= 1e-12 * (bound[i, j] + 1)


def test_unit_scales_reduce_to_the_mxfp4_dequantizer():
    """Block scale e4m3 1.0 (0x38) and global 1: the E2M1 values themselves,
    as the MXFP4 dequantizer gives them under E8M0 127 (= 1.0)."""
    _, codes, _, _ = wl.nvfp4_weight(1, 96, 7, seed=5)
    ones = np.full((7, 96 // 16), 0x38, np.uint8)
    w = oracle.dequant_nvfp4(codes, ones, 1.0)
    w_mx = oracle.mxfp4_dequant(codes, np.full((7, 96 // 32), 127, np.uint8))
    assert np.array_equal(w, w_mx)


def test_block_width_is_sixteen_and_local():
    """Changing block scale (n, b) rescales exactly W_deq[n, 16b:16b+16]."""
    _, codes, scales, g = wl.nvfp4_weight(1, 128, 4, seed=6)
    w0 = oracle.dequant_nvfp4(codes, scales, g)
    s2 = scales.copy()
    s2[2, 3] = 0x48                  # 2^(9-7) = 4.0
    w1 = oracle.dequant_nvfp4(codes, s2, g)
    diff = w1 != w0
    diff[2, 48:64] = False
    assert not diff.any()
    old = float(oracle.e4m3fn_decode(np.array([scales[2, 3]], np.uint8))[0])
    assert np.array_equal(w1[2, 48:64], w0[2, 48:64] * (4.0 / old))


def test_rejects_nan_scales_and_bad_shapes():
    _, codes, scales, g = wl.nvfp4_weight(1, 64, 2, seed=7)
    bad = scales.copy()
    bad[0, 0] = 0x7F
    with pytest.raises(ValueError):
        oracle.dequant_nvfp4(codes, bad, g)
    with pytest.raises(ValueError):
        oracle.dequant_nvfp4(codes, scales[:, :2], g)
