"""Seeded synthetic inputs for the quantized GEMM workloads.

This module only draws random numbers in the shapes and distributions of the
workloads; it performs none of the quantization or GEMM arithmetic.  It is the
one piece shared by the oracle-side tests and the GPU-side tests/benchmark.

Every generator draws its tensors in the order listed from
``numpy.random.default_rng(seed)`` on the host.

Workloads (sizes and distributions):

* ``w4a16_small``  -- W4A16, M=16, K=N=1024.  X fp16 ~ N(0,1); packed INT4
  weights [K/2, N] uint8 (two codes per byte, uniform 0..15 each, so the byte
  is uniform 0..255); per-column fp16 scale ~ U[0.005, 0.02].
* ``w8a16_decode`` -- W8A16, M in {1,4,16}, K=4096, N=11008.  X fp16 ~ N(0,1);
  W int8 [K, N] uniform -127..127; per-column fp16 scale ~ U[0.002, 0.01].
* ``w4a16_decode`` -- W4A16, M in {1,8,16}, K=8192, N=28672, drawn as
  ``w4a16_small``.
* ``mxfp4_square`` -- MXFP4 x MXFP4, M=N=K=8192.  A [M,K] and W [N,K] fp32 ~
  N(0, 0.5^2), to be quantized per 32-element block.
* ``fp8_square``   -- FP8 e4m3fn, M=N=K=8192 (plus an M=16 decode batch).
  A [M,K] and B [K,N] fp32 ~ N(0,1), to be scaled per tensor and cast.

The W8A16 page's own test (M,N,K = 32,256,128) draws W from -128..126 and
scales from N(0,1)*0.01; ``w8a16_page_test`` reproduces that distribution
(negative scales and the -128 code included).
"""

from dataclasses import dataclass

import numpy as np

SEED = 0


@dataclass(frozen=True)
class Workload:
    name: str
    fmt: str
    ms: tuple
    n: int
    k: int


WORKLOADS = {
    "w4a16_small": Workload("w4a16_small", "w4a16", (16,), 1024, 1024),
    "w8a16_decode": Workload("w8a16_decode", "w8a16", (1, 4, 16), 11008, 4096),
    "w4a16_decode": Workload("w4a16_decode", "w4a16", (1, 8, 16), 28672, 8192),
    "mxfp4_square": Workload("mxfp4_square", "mxfp4", (8192,), 8192, 8192),
    "fp8_square": Workload("fp8_square", "fp8", (8192, 16), 8192, 8192),
}


def _normal_f16(rng, shape):
    return rng.standard_normal(shape, dtype=np.float32).astype(np.float16)


def w4a16(m, k, n, seed=SEED):
    """(x fp16 [m,k], packed uint8 [k/2,n], scales fp16 [n])."""
    if k % 2:
        raise ValueError("K must be even for two codes per byte")
    rng = np.random.default_rng(seed)
    x = _normal_f16(rng, (m, k))
    packed = rng.integers(0, 256, size=(k // 2, n), dtype=np.uint8)
    scales = rng.uniform(0.005, 0.02, size=n).astype(np.float16)
    return x, packed, scales


def w8a16(m, k, n, seed=SEED):
    """(x fp16 [m,k], w int8 [k,n] in -127..127, scales fp16 [n])."""
    rng = np.random.default_rng(seed)
    x = _normal_f16(rng, (m, k))
    w = rng.integers(-127, 128, size=(k, n), dtype=np.int8)
    scales = rng.uniform(0.002, 0.01, size=n).astype(np.float16)
    return x, w, scales


def _cdiv(a, b):
    return -(-a // b)


def w4a16_grouped(m, k, n, group_k, group_n=1, zeros=True, seed=SEED):
    """(x fp16 [m,k], packed uint8 [k/2,n], scales fp16 [ceil(k/gk), ceil(n/gn)],
    zero points uint8 0..15 of the same shape, or None)."""
    if k % 2:
        raise ValueError("K must be even for two codes per byte")
    rng = np.random.default_rng(seed)
    x = _normal_f16(rng, (m, k))
    packed = rng.integers(0, 256, size=(k // 2, n), dtype=np.uint8)
    shape = (_cdiv(k, group_k), _cdiv(n, group_n))
    scales = rng.uniform(0.005, 0.02, size=shape).astype(np.float16)
    z = rng.integers(0, 16, size=shape, dtype=np.uint8) if zeros else None
    return x, packed, scales, z


def w8a16_grouped(m, k, n, group_k, group_n=1, zeros=True, seed=SEED):
    """(x fp16 [m,k], w int8 [k,n] in -127..127, scales fp16 [ceil(k/gk),
    ceil(n/gn)], zero points int8 -32..32 of the same shape, or None)."""
    rng = np.random.default_rng(seed)
    x = _normal_f16(rng, (m, k))
    w = rng.integers(-127, 128, size=(k, n), dtype=np.int8)
    shape = (_cdiv(k, group_k), _cdiv(n, group_n))
    scales = rng.uniform(0.002, 0.01, size=shape).astype(np.float16)
    z = rng.integers(-32, 33, size=shape, dtype=np.int8) if zeros else None
    return x, w, scales, z


def nvfp4_weight(m, k, n, seed=SEED):
    """(x fp16 [m,k], codes uint8 [n,k/2], block scales uint8 e4m3 [n,k/16],
    global fp32).  Codes: uniform bytes.  Block scales: positive normal e4m3
    with exponent field 4..10 (values 2^-3 .. 2^3 * (1 + m/8)).  The global
    scale 0.01 keeps |Y| of order one."""
    rng = np.random.default_rng(seed)
    x = _normal_f16(rng, (m, k))
    codes = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    exp = rng.integers(4, 11, size=(n, k // 16))
    man = rng.integers(0, 8, size=(n, k // 16))
    scales = ((exp << 3) | man).astype(np.uint8)
    return x, codes, scales, np.float32(0.01)


def w8a16_page_test(m=32, k=128, n=256, seed=SEED):
    """The W8A16 page's test distribution: w in -128..126, scales N(0,1)*0.01."""
    rng = np.random.default_rng(seed)
    x = _normal_f16(rng, (m, k))
    w = rng.integers(-128, 127, size=(k, n), dtype=np.int8)
    scales = (rng.standard_normal(n, dtype=np.float32) * np.float32(0.01)).astype(np.float16)
    return x, w, scales


def mxfp4_operands(m, n, k, seed=SEED, sigma=0.5):
    """(a fp32 [m,k], w fp32 [n,k]) ~ N(0, sigma^2)."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((m, k), dtype=np.float32) * np.float32(sigma)
    w = rng.standard_normal((n, k), dtype=np.float32) * np.float32(sigma)
    return a, w


def fp8_operands(m, n, k, seed=SEED):
    """(a fp32 [m,k], b fp32 [k,n]) ~ N(0, 1)."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((m, k), dtype=np.float32)
    b = rng.standard_normal((k, n), dtype=np.float32)
    return a, b


def sample_indices(m, n, count, seed=SEED + 1):
    """`count` distinct-ish (row, col) output positions for sampled checks,
    always including the four corners."""
    rng = np.random.default_rng(seed)
    rows = rng.integers(0, m, size=count)
    cols = rng.integers(0, n, size=count)
    rows[:4] = [0, 0, m - 1, m - 1]
    cols[:4] = [0, n - 1, 0, n - 1]
    return rows, cols
