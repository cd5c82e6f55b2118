"""Quantizers: MXFP4 (E2M1 + E8M0 per 32-element block) and per-tensor FP8.

TEST INFRASTRUCTURE (oracle).  Importable only by the tests, the smoke check
and the benchmark's CPU-baseline leg.

Parity pins (tests/test_oracle_pins.py): exponent-rule invariants, brute-force
nearest-grid search in exact rationals, every tie point and its one-ulp
neighbours, and the page's own fp32 torch formulation on random blocks.  The
FP8 scale formula is parity unpinned (see the package docstring); its encoder
is pinned to the e4m3fn definition and to torch's float8_e4m3fn cast.
"""

import numpy as np

from .formats import (
    E2M1_GRID,
    pack_nibbles_last_axis,
    unpack_nibbles_last_axis,
    e2m1_decode,
    e8m0_decode,
    e4m3fn_encode,
)

MICRO_BLOCK = 32          # MXFP4 page, intro and section 2: 32 elements per block
E2M1_MAX = 6.0            # largest grid magnitude
AMAX_FLOOR = np.float32(1e-8)   # MXFP4 page section 3: block maxima clamped below
E4M3_MAX = 448.0          # FP8 page, precision management: scale_max = 448


def mxfp4_quantize(x):
    """fp32 [R, K] -> (codes [R, K/2] uint8, e8m0 [R, K/32] uint8).

    Steps, in the order of the MXFP4 page's section-3 simulator:
      1. split each row into blocks of 32 along K;
      2. amax = max |x| over the block, clamped to at least 1e-8 (as fp32);
      3. shared exponent e = ceil(log2(amax / 6)), stored biased as E = e + 127;
      4. divide the block by 2**e (exact);
      5. each magnitude goes to the nearest grid point of E2M1_GRID, the first
         (smaller) one on a tie, since the simulator takes argmin over the grid;
      6. the element keeps the sign of x; a negative value that rounds to zero
         keeps its sign bit (the simulator multiplies sign(x) into the grid
         value, and sign(-0.0) is +0).
    Codes are sign<<3 | grid index, two per byte, even element in the low nibble.
    """
    x = np.asarray(x)
    if x.dtype != np.float32 or x.ndim != 2:
        raise ValueError("mxfp4_quantize takes a 2-D float32 array")
    rows, k = x.shape
    if k % MICRO_BLOCK:
        raise ValueError("K must be a multiple of 32")
    if not np.all(np.isfinite(x)):
        raise ValueError("inputs must be finite")
    blocks = x.reshape(rows, k // MICRO_BLOCK, MICRO_BLOCK).astype(np.float64)

    amax = np.abs(blocks).max(axis=-1)
    amax = np.maximum(amax, np.float64(AMAX_FLOOR))
    e = np.ceil(np.log2(amax / E2M1_MAX)).astype(np.int64)
    big_e = e + 127
    if big_e.min(initial=127) < 0 or big_e.max(initial=127) > 254:
        raise ValueError("block exponent outside the E8M0 range")

    normalized = blocks / np.ldexp(1.0, e)[..., None]
    dist = np.abs(np.abs(normalized)[..., None] - E2M1_GRID)
    idx = np.argmin(dist, axis=-1)            # first minimum wins a tie
    sign_bit = (blocks < 0).astype(np.int64)
    codes = (sign_bit << 3) | idx
    codes = codes.reshape(rows, k)
    return pack_nibbles_last_axis(codes), big_e.astype(np.uint8)


def mxfp4_dequant(codes_packed, e8m0):
    """(codes [R, K/2], e8m0 [R, K/32]) -> fp64 [R, K]: element * 2**(E - 127).

    MXFP4 page, section 2 eq. (1): each block's elements carry their block scale.
    """
    vals = e2m1_decode(unpack_nibbles_last_axis(codes_packed))
    rows, k = vals.shape
    e8m0 = np.asarray(e8m0)
    if e8m0.shape != (rows, k // MICRO_BLOCK):
        raise ValueError("scale array must be [rows, K/32]")
    scale = np.repeat(e8m0_decode(e8m0), MICRO_BLOCK, axis=1)
    return vals * scale


def fp8_quantize(x):
    """fp32 tensor -> (e4m3fn codes uint8 of the same shape, fp32 scale).

    FP8 page, precision management: per-tensor scaling so that the tensor fits
    the e4m3fn range of +-448.  Reading (the page gives no formula): scale =
    fp32(max|x| / 448); code = e4m3fn(fp32(x / scale)) with round-to-nearest-
    even and saturation at 448; an all-zero tensor gets scale 1.
    """
    x = np.asarray(x)
    if x.dtype != np.float32:
        raise ValueError("fp8_quantize takes float32 input")
    if not np.all(np.isfinite(x)):
        raise ValueError("inputs must be finite")
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0)
    if amax == 0:
        scale = np.float32(1.0)
    else:
        scale = np.float32(amax / np.float32(E4M3_MAX))   # fp32 division
    v = (x / scale).astype(np.float32)                    # fp32 division
    return e4m3fn_encode(v.astype(np.float64)), scale
