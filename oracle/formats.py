"""Bit-level formats of the quantized operands, written from their definitions.

TEST INFRASTRUCTURE (oracle).  Importable only by the tests, the smoke check
and the benchmark's CPU-baseline leg.

Everything here is exact: codes are integers, and every decoded value is a
dyadic rational that fp64 holds exactly.
"""

import numpy as np

# E2M1 magnitudes in index order.  The MXFP4 page, section 3, lists this table
# as the simulator's lookup grid; index i is also the 3-bit exponent/mantissa
# field of an E2M1 code (pinned against the E2M1 closed form in the tests).
E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


# --------------------------------------------------------------------------
# INT4 codes packed two per byte
# --------------------------------------------------------------------------

def unpack_int4_along_k(packed):
    """[K/2, N] uint8 -> [K, N] codes 0..15.

    W4A16 page, section 2 (kernel body): row k of the weight lives in byte row
    k // 2, and the nibble is taken by shifting right by 4 * (k % 2) and masking
    with 0xF, so even k sits in the low nibble and odd k in the high nibble.
    """
    packed = np.asarray(packed)
    if packed.dtype != np.uint8 or packed.ndim != 2:
        raise ValueError("packed INT4 weights must be a 2-D uint8 array")
    half_k, n = packed.shape
    codes = np.empty((2 * half_k, n), dtype=np.uint8)
    for k in range(2):  # k % 2 selects the nibble
        codes[k::2, :] = (packed >> (4 * k)) & 0xF
    return codes


def pack_int4_along_k(codes):
    """[K, N] codes 0..15 -> [K/2, N] uint8; inverse of unpack_int4_along_k."""
    codes = np.asarray(codes)
    if codes.ndim != 2 or codes.shape[0] % 2:
        raise ValueError("need a 2-D code array with an even number of K rows")
    if codes.min(initial=0) < 0 or codes.max(initial=0) > 15:
        raise ValueError("INT4 codes must lie in 0..15")
    c = codes.astype(np.uint8)
    return (c[0::2, :] | (c[1::2, :] << 4)).astype(np.uint8)


def unpack_nibbles_last_axis(packed):
    """[R, C/2] uint8 -> [R, C] codes; element 2j in the low nibble of byte j.

    The MXFP4 page gives no bit layout for its data segment; this build reads
    it the way the W4A16 page packs INT4 (low nibble first along K).
    """
    packed = np.asarray(packed)
    if packed.dtype != np.uint8 or packed.ndim != 2:
        raise ValueError("packed codes must be a 2-D uint8 array")
    r, half_c = packed.shape
    codes = np.empty((r, 2 * half_c), dtype=np.uint8)
    codes[:, 0::2] = packed & 0xF
    codes[:, 1::2] = packed >> 4
    return codes


def pack_nibbles_last_axis(codes):
    """[R, C] codes 0..15 -> [R, C/2] uint8; inverse of unpack_nibbles_last_axis."""
    codes = np.asarray(codes)
    if codes.ndim != 2 or codes.shape[1] % 2:
        raise ValueError("need a 2-D code array with an even number of columns")
    if codes.min(initial=0) < 0 or codes.max(initial=0) > 15:
        raise ValueError("codes must lie in 0..15")
    c = codes.astype(np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


# --------------------------------------------------------------------------
# MXFP4 element and scale
# --------------------------------------------------------------------------

def e2m1_decode(codes):
    """4-bit E2M1 code -> fp64 value: sign bit 3, magnitude index in bits 0..2.

    MXFP4 page, section 3: an element is sign times a grid magnitude.
    """
    codes = np.asarray(codes).astype(np.int64)
    if codes.min(initial=0) < 0 or codes.max(initial=0) > 15:
        raise ValueError("E2M1 codes must lie in 0..15")
    mag = E2M1_GRID[codes & 0x7]
    return np.where(codes & 0x8, -mag, mag)


def e8m0_decode(e):
    """E8M0 byte E -> 2**(E - 127) in fp64 (255 is NaN).

    MXFP4 page, section 2, eq. (2): a scale is a pure power of two with bias 127.
    """
    e = np.asarray(e).astype(np.int64)
    if e.min(initial=0) < 0 or e.max(initial=0) > 255:
        raise ValueError("E8M0 scales are bytes")
    val = np.ldexp(1.0, e - 127)
    return np.where(e == 255, np.nan, val)


# --------------------------------------------------------------------------
# FP8 E4M3 (the "fn" variant: no infinities, one NaN pattern per sign, max 448)
# --------------------------------------------------------------------------

def e4m3fn_decode(codes):
    """uint8 e4m3fn code -> fp64.

    FP8 page, precision management: inputs are e4m3fn with range +-448.  The
    format has exponent bias 7, three mantissa bits, subnormals at exponent
    field 0 and S.1111.111 as NaN (no infinities).
    """
    c = np.asarray(codes).astype(np.int64)
    if c.min(initial=0) < 0 or c.max(initial=0) > 255:
        raise ValueError("e4m3fn codes are bytes")
    sign = np.where(c & 0x80, -1.0, 1.0)
    exp = (c >> 3) & 0xF
    man = (c & 0x7).astype(np.float64)
    normal = np.ldexp(1.0 + man / 8.0, exp - 7)
    subnormal = np.ldexp(man / 8.0, -6)
    mag = np.where(exp == 0, subnormal, normal)
    mag = np.where((exp == 15) & ((c & 0x7) == 7), np.nan, mag)
    return sign * mag


def e4m3fn_encode(x):
    """fp64/fp32 value -> e4m3fn code, round to nearest, ties to even, and
    saturating at +-448 (never produces the NaN pattern for finite input).

    The FP8 page states no rounding mode; this is IEEE round-to-nearest-even
    with saturation, which is what an exact cast of values up to 448 gives.
    Inputs must be finite.
    """
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("e4m3fn_encode needs finite input")
    sign = np.signbit(x)
    v = np.abs(x)
    # exponent of the binade holding v, clamped to the smallest normal (2**-6);
    # below it the spacing stays 2**-9 (subnormals)
    _, e2 = np.frexp(np.where(v > 0, v, 1.0))  # v = f * 2**e2, f in [0.5, 1)
    unbiased = np.maximum(e2 - 1, -6)
    quantum = np.ldexp(1.0, unbiased - 3)
    q = np.rint(v / quantum) * quantum  # rint rounds half to even
    q = np.minimum(q, 448.0)
    # re-derive the bit fields of q
    _, e2q = np.frexp(np.where(q > 0, q, 1.0))
    uq = e2q - 1
    is_sub = (q < 2.0 ** -6)
    exp_field = np.where(is_sub, 0, uq + 7)
    man_field = np.where(
        is_sub,
        np.rint(q / 2.0 ** -9),
        np.rint((q / np.ldexp(1.0, uq) - 1.0) * 8.0),
    )
    code = (exp_field.astype(np.int64) << 3) | man_field.astype(np.int64)
    code = np.where(sign, code | 0x80, code)
    return code.astype(np.uint8)


# --------------------------------------------------------------------------
# Output casts (fp32 accumulator -> low precision store)
# --------------------------------------------------------------------------

def round_fp16(x):
    """Round to the nearest fp16, ties to even; returns fp64 values.

    W4A16 page section 2 and W8A16 page solution: the fp32 accumulator is cast
    to fp16 on store.  NumPy's double->half conversion is correctly rounded.
    """
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def round_bf16(x):
    """Round to the nearest bf16 (8 significant bits), ties to even; fp64 out.

    FP8 page, precision management: the output is stored as bf16.  Values are
    assumed to lie in the normal bf16 range (true for every workload here).
    """
    x = np.asarray(x, dtype=np.float64)
    f, e = np.frexp(x)  # x = f * 2**e, |f| in [0.5, 1)
    return np.ldexp(np.rint(f * 256.0), e - 8)
