"""The dispatch rules, asked of the library (host-only, no GPU needed).

qgemm_dispatch_kernel answers from the same function every GEMM entry point
uses to choose its kernel.  These cases pin each edge of the rules:

* weight-only formats (INT4, INT8, grouped, NVFP4): the 256 x 256 tile
  kernel from M = 256 once T = ceil(M/256) * ceil(N/256) >= 192, or from
  M = 640 once T >= 48; fp16 rows with K % 8 != 0 and empty K stay on the
  small-M kernel;
* FP8 / MXFP4: the small-M kernel up to M = 64; 65 .. 128 rows unless N is
  wide (FP8 >= 24576, MXFP4 >= 16384); above, FP8 up to M = 512 while
  M * N <= 2621440 and MXFP4 up to M = 256 while M * N <= 2^21; otherwise
  256 x 256 tiles (M > 64, N > 128, K of at least two 128-element tiles,
  MXFP4 K a multiple of 128 and at least two 256-element steps) or 128 x 128
  tiles;
* operands whose packed bytes reach 2^31 leave the 256 x 256 kernels.

The GPU parity tests run shapes on both sides of the same edges.
"""

import pytest

import bit_quantized_gemm_qgemm_amd as qg

SMALL, WO, MX, F8, T128 = ("decode_gemm_kernel", "pipe256_kernel", "mxw_kernel", "f8w_kernel",
                           "tile_gemm_kernel")


@pytest.fixture(scope="module", autouse=True)
def library():
    return qg.lib()   # the built library (host code only is exercised)


@pytest.mark.parametrize("fmt", ["w4a16", "w8a16", "nvfp4"])
@pytest.mark.parametrize("m,n,k,want", [
    (16, 11008, 4096, SMALL),
    (255, 65536, 4096, SMALL),     # M < 256
    (256, 24576, 256, SMALL),      # T = 96
    (257, 24576, 256, WO),         # T = 192
    (639, 12288, 256, SMALL),      # T = 144, M < 640
    (640, 12288, 256, WO),         # M >= 640, T >= 48
    (1024, 2816, 256, SMALL),      # T = 44
    (1280, 2560, 256, WO),         # T = 50
    (4096, 128, 4096, SMALL),      # N <= 128
    (4096, 4096, 4096, WO),
    (0, 4096, 4096, None),
    (4096, 0, 4096, None),
])
def test_weight_only_rule(fmt, m, n, k, want):
    assert qg.qgemm_dispatch_kernel(fmt, m, n, k) == want


def test_weight_only_edges_of_k():
    assert qg.qgemm_dispatch_kernel("w8a16", 4096, 4096, 4100) == SMALL   # K % 8 != 0
    assert qg.qgemm_dispatch_kernel("w8a16", 4096, 4096, 0) == SMALL      # empty K
    assert qg.qgemm_dispatch_kernel("w4a16", 4096, 4096, 4104) == WO      # K % 8 == 0


@pytest.mark.parametrize("fmt", ["w4a16_grouped", "w8a16_grouped"])
def test_grouped_rule(fmt):
    assert qg.qgemm_dispatch_kernel(fmt, 256, 24576, 256, 64) == SMALL
    assert qg.qgemm_dispatch_kernel(fmt, 257, 24576, 256, 64) == WO
    assert qg.qgemm_dispatch_kernel(fmt, 16, 28672, 8192, 128) == SMALL
    assert qg.qgemm_dispatch_kernel(fmt, 4096, 4096, 4096, 128) == WO


@pytest.mark.parametrize("m,n,k,want", [
    (1, 8192, 8192, SMALL),
    (64, 28672, 8192, SMALL),      # M <= 64
    (65, 28672, 8192, F8),         # 65 .. 128 rows, wide N
    (128, 24560, 256, SMALL),      # N < 24576
    (128, 24576, 256, F8),
    (100, 24600, 128, T128),       # one 128-element K tile
    (129, 20320, 256, SMALL),      # M * N <= 2621440
    (129, 20336, 256, F8),
    (512, 5120, 1024, SMALL),
    (512, 5136, 1024, F8),
    (513, 64, 272, T128),          # M > 512, N <= 128
    (8192, 8192, 8192, F8),
])
def test_fp8_rule(m, n, k, want):
    assert qg.qgemm_dispatch_kernel("fp8", m, n, k) == want


@pytest.mark.parametrize("m,n,k,want", [
    (16, 8192, 8192, SMALL),
    (64, 28672, 8192, SMALL),
    (65, 17000, 640, MX),          # 65 .. 128 rows, wide N
    (128, 16368, 512, SMALL),      # N < 16384
    (128, 16384, 512, MX),
    (100, 16400, 288, T128),       # K not a multiple of 128
    (100, 16400, 256, T128),       # one 256-element step
    (256, 8192, 512, SMALL),       # M * N = 2^21
    (256, 8208, 512, MX),
    (257, 200, 640, MX),           # M > 256
    (8192, 8192, 8192, MX),
])
def test_mxfp4_rule(m, n, k, want):
    assert qg.qgemm_dispatch_kernel("mxfp4", m, n, k) == want


def test_operands_past_2gib_leave_the_256_tiles():
    # packed FP8 B of K * N >= 2^31 bytes: the 128 x 128 kernel (64-bit addressing)
    assert qg.qgemm_dispatch_kernel("fp8", 256, 32832, 65536) == T128
    assert qg.qgemm_dispatch_kernel("mxfp4", 256, 61696, 65536) == T128
    # a weight-only X of 2^31 bytes or more keeps the small-M kernel
    assert qg.qgemm_dispatch_kernel("w8a16", 262144, 4096, 4096) == SMALL


def test_rejected_arguments():
    with pytest.raises(qg.QgemmError):
        qg.qgemm_dispatch_kernel(99, 4, 4, 32)
    with pytest.raises(qg.QgemmError):
        qg.qgemm_dispatch_kernel("mxfp4", 4, 4, 40)          # K % 32 != 0
    with pytest.raises(qg.QgemmError):
        qg.qgemm_dispatch_kernel("w4a16_grouped", 4, 4, 64, 48)   # group not a multiple of 32
    with pytest.raises(qg.QgemmError):
        qg.qgemm_dispatch_kernel("fp8", -1, 4, 32)
