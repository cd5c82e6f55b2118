"""CPU oracle for the four on-the-fly-dequantizing GEMM variants.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test-suite, the package's
smoke check and the CPU-baseline leg of the benchmark may import this package.
It shares no code with the HIP library: it dequantizes every operand to fp64
exactly and multiplies with NumPy, as plainly as the method can be written.

Sources (the web pages these functions restate; short names used below):

* "W4A16 page"  -- Triton W4A16 blocked GEMM and Blackwell NVFP4 instructions
  (dreamvfia.cn, research/triton-w4a16-blackwell-nvfp4), sections 1-3.
* "MXFP4 page"  -- MXFP4 matrix-multiplication kernel principle
  (pwwt.cn, news/5064028), sections 1-3 with eq. (1) block dot product and
  eq. (2) exponent-add scale product.
* "W8A16 page"  -- Triton quantization: W8A16 weight-quantized fused GEMM
  (datawhalechina llm-algo-leetcode, chapter 10), Steps 1-4 and the solution.
* "FP8 page"    -- FP8 GEMM kernel in Triton via CUTLASS naming
  (blog.hotdry.top, 2025/10/03), kernel example and parameter list.

Group-wise scales and zero points (grouped.py) follow the W4A16 page's
section 1 dequant form and the W8A16 page's extensions; NVFP4-style two-level
block scaling (nvfp4.py) the W4A16 page's section 3.

Parity status of each function is stated in its module.  Parity unpinned:
the FP8 per-tensor scale formula (the FP8 page fixes only the 448 range and
per-tensor scaling; GEMM parity is taken against the quantized operands, so
only the scale's properties are pinned).
"""

from .formats import (
    E2M1_GRID,
    unpack_int4_along_k,
    pack_int4_along_k,
    unpack_nibbles_last_axis,
    pack_nibbles_last_axis,
    e2m1_decode,
    e8m0_decode,
    e4m3fn_decode,
    e4m3fn_encode,
    round_fp16,
    round_bf16,
)
from .quantize import mxfp4_quantize, mxfp4_dequant, fp8_quantize
from .nvfp4 import NVFP4_BLOCK, dequant_nvfp4, gemm_nvfp4
from .grouped import (
    expand_groups,
    dequant_w4_grouped,
    dequant_w8_grouped,
    gemm_w4a16_grouped,
    gemm_w8a16_grouped,
)
from .gemm import (
    dequant_w4,
    dequant_w8,
    gemm_w4a16,
    gemm_w8a16,
    gemm_mxfp4,
    gemm_fp8,
    tolerance,
    within_tolerance,
)

__all__ = [
    "E2M1_GRID",
    "unpack_int4_along_k",
    "pack_int4_along_k",
    "unpack_nibbles_last_axis",
    "pack_nibbles_last_axis",
    "e2m1_decode",
    "e8m0_decode",
    "e4m3fn_decode",
    "e4m3fn_encode",
    "round_fp16",
    "round_bf16",
    "mxfp4_quantize",
    "mxfp4_dequant",
    "fp8_quantize",
    "dequant_w4",
    "dequant_w8",
    "gemm_w4a16",
    "gemm_w8a16",
    "gemm_mxfp4",
    "gemm_fp8",
    "tolerance",
    "within_tolerance",
    "expand_groups",
    "dequant_w4_grouped",
    "dequant_w8_grouped",
    "gemm_w4a16_grouped",
    "gemm_w8a16_grouped",
    "NVFP4_BLOCK",
    "dequant_nvfp4",
    "gemm_nvfp4",
]
