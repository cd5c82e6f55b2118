"""NVFP4-style two-level block scaling for the weight operand.

TEST INFRASTRUCTURE (oracle).  Importable only by the tests, the smoke check
and the benchmark's CPU-baseline leg.

Source: W4A16 page, section 3: NVFP4 stores E2M1 elements under a two-level,
block-adaptive scale (a local FP8/FP4 block scale on top of the elements) and
the tensor cores consume it directly.

Readings (the page fixes neither the block size nor the scale formats):
* first level: one E4M3 (e4m3fn, the FP8 page's format) scale per 16
  consecutive K elements of a weight row;
* second level: one fp32 scale for the whole tensor;
* layout as for MXFP4 weights: codes uint8 [N, K/2] with element 2j in the
  low nibble of byte j, block scales uint8 [N, K/16];
* activations fp16 X [M, K], output Y = X @ W_deq^T (fp16 on the device).
W_deq[n, k] = e2m1(code) * e4m3(scale[n, k // 16]) * global, kept exact in
fp64.  NaN block-scale codes (0x7f, 0xff) are rejected.

Pinned in tests/test_oracle_nvfp4.py: exact rational brute force from the bit
fields, reduction to the MXFP4 dequantizer at unit scales, block locality and
the 16-element block width.
"""

import numpy as np

from .formats import e2m1_decode, e4m3fn_decode, unpack_nibbles_last_axis

NVFP4_BLOCK = 16


def dequant_nvfp4(codes, scales, global_scale):
    """codes uint8 [N, K/2], scales uint8 e4m3 [N, K/16], fp32 global -> fp64 [N, K]."""
    c = np.asarray(codes)
    s = np.asarray(scales)
    if c.dtype != np.uint8 or s.dtype != np.uint8 or c.ndim != 2 or s.ndim != 2:
        raise ValueError("codes and scales are 2-D uint8 arrays")
    n, half_k = c.shape
    k = 2 * half_k
    if k % NVFP4_BLOCK or s.shape != (n, k // NVFP4_BLOCK):
        raise ValueError("scales must be [N, K/16] with K a multiple of 16")
    if ((s & 0x7F) == 0x7F).any():
        raise ValueError("NaN block scale")
    elem = e2m1_decode(unpack_nibbles_last_axis(c))                 # [N, K]
    block = np.repeat(e4m3fn_decode(s), NVFP4_BLOCK, axis=1)        # [N, K]
    return elem * block * float(np.float32(global_scale))


def gemm_nvfp4(x, codes, scales, global_scale):
    """(Y = X @ W_deq^T, bound = |X| @ |W_deq|^T) in fp64 for fp16 X [M, K]."""
    wd = dequant_nvfp4(codes, scales, global_scale)
    xd = np.asarray(x).astype(np.float64)
    return xd @ wd.T, np.abs(xd) @ np.abs(wd).T
