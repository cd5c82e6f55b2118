"""Host-side tests of the C ABI: the library loads, exports every entry point
the header declares, and rejects bad arguments before touching a device.

No test here launches a kernel.  If libqgemm.so has not been built yet, it is
built once (hipcc cross-compiles for gfx950 without a GPU).
"""

import ctypes
import os
import re

import pytest

import bit_quantized_gemm_qgemm_amd as qg
from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "qgemm.h")

OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_ARCH, ERR_LAUNCH, ERR_FORMAT, ERR_DEVICE = (
    0, -1, -2, -3, -4, -5, -6, -7)
ERR_TOO_LARGE = -8


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(qg.LIB_PATH):
        from bit_quantized_gemm_qgemm_amd import build
        build.build()
    return qg.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qgemm_\w+)\s*\(", text)))


def test_header_declares_the_expected_entry_points():
    names = declared_functions()
    for want in ("qgemm_w4a16", "qgemm_w8a16", "qgemm_mxfp4", "qgemm_fp8", "qgemm_prepack",
                 "qgemm_prepack_bytes", "qgemm_quantize_mxfp4", "qgemm_quantize_fp8",
                 "qgemm_status_string", "qgemm_abi_version", "qgemm_prepack_grouped",
                 "qgemm_prepack_grouped_bytes", "qgemm_w4a16_grouped", "qgemm_w8a16_grouped",
                 "qgemm_nvfp4", "qgemm_act_workspace_bytes", "qgemm_mxfp4_act",
                 "qgemm_fp8_act", "qgemm_fp8_act_noalloc", "qgemm_dispatch_kernel"):
        assert want in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    # and the binding wraps each of them
    bound = {n for n, _, _ in qg._SIGNATURES}
    assert bound == set(declared_functions())


def test_status_strings(lib):
    for st in (OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_ARCH, ERR_LAUNCH, ERR_FORMAT, ERR_DEVICE,
               ERR_TOO_LARGE):
        s = qg.status_string(st)
        assert s and s != "unknown status"
    assert qg.status_string(12345) == "unknown status"
    assert lib.qgemm_abi_version() == 103


def test_prepack_bytes(lib):
    # W4A16 at K = N = 1024: 64 column groups x 8 K-tiles x 1 KB, no padding
    assert lib.qgemm_prepack_bytes(1, 1024, 1024) == 1024 * 1024 // 2
    # W4A16 at K = 8192, N = 28672: exactly the canonical 117,440,512 bytes
    assert lib.qgemm_prepack_bytes(1, 8192, 28672) == 8192 * 28672 // 2
    assert lib.qgemm_prepack_bytes(2, 4096, 11008) == 4096 * 11008
    assert lib.qgemm_prepack_bytes(4, 8192, 8192) == 8192 * 8192
    # MXFP4: code segment + 256-aligned scale segment (one byte per 32 elements)
    assert lib.qgemm_prepack_bytes(3, 8192, 8192) == 8192 * 8192 // 2 + 8192 * 8192 // 32
    # ragged sizes round up to whole 16-column x K tiles
    assert lib.qgemm_prepack_bytes(2, 130, 17) == 2 * 2 * 2048
    assert lib.qgemm_prepack_bytes(1, 0, 5) == 0
    assert lib.qgemm_prepack_bytes(1, 3, 5) == ERR_SHAPE      # odd K for W4
    assert lib.qgemm_prepack_bytes(3, 48, 5) == ERR_SHAPE     # K % 32 for MXFP4
    assert lib.qgemm_prepack_bytes(4, 24, 5) == ERR_SHAPE     # K % 16 for FP8
    assert lib.qgemm_prepack_bytes(9, 32, 32) == ERR_FORMAT
    assert lib.qgemm_prepack_bytes(2, -1, 5) == ERR_SHAPE


P = ctypes.c_void_p
GOOD = P(0x10000)      # 16-byte aligned, never dereferenced by these calls
ODD = P(0x10008)       # 8-byte aligned only


def test_gemm_argument_errors_need_no_device(lib):
    s = P(0)
    for fn in (lib.qgemm_w4a16, lib.qgemm_w8a16):
        assert fn(None, GOOD, GOOD, GOOD, 4, 4, 32, s) == ERR_NULL
        assert fn(None, None, GOOD, None, 4, 4, 0, s) == ERR_NULL   # Y still has 16 elements
        assert fn(None, None, GOOD, GOOD, 4, 4, 0, s) != ERR_NULL   # K = 0: X, W empty
        assert fn(GOOD, GOOD, GOOD, GOOD, -1, 4, 32, s) == ERR_SHAPE
        assert fn(GOOD, ODD, GOOD, GOOD, 4, 4, 32, s) == ERR_ALIGN
        assert fn(GOOD, GOOD, GOOD, GOOD, 0, 4, 32, s) == OK      # empty: no-op
        assert fn(GOOD, GOOD, GOOD, GOOD, 4, 0, 32, s) == OK
    assert lib.qgemm_w4a16(GOOD, GOOD, GOOD, GOOD, 4, 4, 31, s) == ERR_SHAPE
    assert lib.qgemm_w8a16(GOOD, GOOD, GOOD, GOOD, 0, 4, 31, s) == OK
    assert lib.qgemm_w8a16(None, GOOD, GOOD, None, 0, 4, 31, s) == OK   # empty X and Y
    assert lib.qgemm_mxfp4(GOOD, GOOD, None, GOOD, 4, 4, 32, s) == ERR_NULL
    assert lib.qgemm_mxfp4(GOOD, GOOD, GOOD, GOOD, 4, 4, 48, s) == ERR_SHAPE
    assert lib.qgemm_mxfp4(GOOD, GOOD, GOOD, ODD, 4, 4, 64, s) == ERR_ALIGN
    assert lib.qgemm_mxfp4(GOOD, GOOD, GOOD, GOOD, 0, 4, 64, s) == OK
    assert lib.qgemm_fp8(GOOD, GOOD, None, GOOD, GOOD, 4, 4, 32, s) == ERR_NULL
    assert lib.qgemm_fp8(GOOD, GOOD, GOOD, GOOD, GOOD, 4, 4, 40, s) == ERR_SHAPE
    assert lib.qgemm_fp8(GOOD, GOOD, P(0x10002), GOOD, GOOD, 4, 4, 32, s) == ERR_ALIGN
    assert lib.qgemm_fp8(GOOD, GOOD, GOOD, GOOD, GOOD, 4, 0, 32, s) == OK
    # sizes whose element offsets would overflow the kernels' 32-bit indexing
    assert lib.qgemm_w8a16(GOOD, GOOD, GOOD, GOOD, 1 << 20, 1 << 20, 64, s) == ERR_SHAPE


def test_prepack_and_quantize_argument_errors(lib):
    s = P(0)
    assert lib.qgemm_prepack(9, GOOD, None, GOOD, 32, 32, s) == ERR_FORMAT
    assert lib.qgemm_prepack(5, GOOD, None, GOOD, 32, 32, s) == ERR_FORMAT   # grouped: own prepack
    assert lib.qgemm_prepack(1, GOOD, None, None, 32, 32, s) == ERR_NULL
    assert lib.qgemm_prepack(1, None, None, GOOD, 32, 32, s) == ERR_NULL
    assert lib.qgemm_prepack(3, GOOD, None, GOOD, 64, 32, s) == ERR_NULL   # MXFP4 needs scales
    assert lib.qgemm_prepack(1, GOOD, None, ODD, 32, 32, s) == ERR_ALIGN
    assert lib.qgemm_prepack(1, GOOD, None, GOOD, 33, 32, s) == ERR_SHAPE
    assert lib.qgemm_prepack(2, None, None, GOOD, 0, 32, s) == OK          # nothing to pack
    assert lib.qgemm_quantize_mxfp4(None, 4, 32, GOOD, GOOD, s) == ERR_NULL
    assert lib.qgemm_quantize_mxfp4(GOOD, 4, 48, GOOD, GOOD, s) == ERR_SHAPE
    assert lib.qgemm_quantize_mxfp4(ODD, 4, 32, GOOD, GOOD, s) == ERR_ALIGN
    assert lib.qgemm_quantize_mxfp4(GOOD, 0, 32, GOOD, GOOD, s) == OK
    assert lib.qgemm_quantize_fp8(GOOD, 16, GOOD, None, s) == ERR_NULL
    assert lib.qgemm_quantize_fp8(GOOD, -1, GOOD, GOOD, s) == ERR_SHAPE
    assert lib.qgemm_quantize_fp8(GOOD, 16, GOOD, P(0x10001), s) == ERR_ALIGN


def test_nvfp4_sizes_and_argument_errors(lib):
    s = P(0)
    # W4A16 code geometry (1 KB per 16 x 128 tile), then 128 B of block scales per tile
    assert lib.qgemm_prepack_bytes(7, 8192, 28672) == 8192 * 28672 // 2 + 1792 * 64 * 128
    assert lib.qgemm_prepack_bytes(7, 48, 20) == 2 * 1024 + 2 * 128
    assert lib.qgemm_prepack_bytes(7, 40, 16) == ERR_SHAPE                   # K % 16
    assert lib.qgemm_prepack(7, GOOD, None, GOOD, 64, 32, s) == ERR_NULL     # block scales
    assert lib.qgemm_nvfp4(GOOD, GOOD, None, GOOD, 4, 16, 64, s) == ERR_NULL  # global scale
    assert lib.qgemm_nvfp4(GOOD, GOOD, GOOD, GOOD, 4, 16, 72, s) == ERR_SHAPE
    assert lib.qgemm_nvfp4(GOOD, GOOD, P(0x10002), GOOD, 4, 16, 64, s) == ERR_ALIGN
    assert lib.qgemm_nvfp4(GOOD, ODD, GOOD, GOOD, 4, 16, 64, s) == ERR_ALIGN
    assert lib.qgemm_nvfp4(GOOD, GOOD, GOOD, GOOD, 0, 16, 64, s) == OK


def test_act_workspace_and_argument_errors(lib):
    s = P(0)
    assert lib.qgemm_act_workspace_bytes(3, 16, 8192) == 16 * 8192 // 2 + 16 * 256
    assert lib.qgemm_act_workspace_bytes(3, 3, 96) == 144 + 9      # codes rounded to 16
    assert lib.qgemm_act_workspace_bytes(4, 16, 8192) == 16 * 8192 + 16 + 1024   # + partial maxima
    assert lib.qgemm_act_workspace_bytes(4, 3, 16) == 48 + 16 + 1024
    assert lib.qgemm_act_workspace_bytes(1, 16, 64) == ERR_FORMAT
    assert lib.qgemm_act_workspace_bytes(3, 16, 48) == ERR_SHAPE
    assert lib.qgemm_mxfp4_act(GOOD, GOOD, GOOD, None, 4, 16, 64, s) == ERR_NULL
    assert lib.qgemm_mxfp4_act(GOOD, GOOD, GOOD, ODD, 4, 16, 64, s) == ERR_ALIGN
    assert lib.qgemm_mxfp4_act(GOOD, GOOD, GOOD, GOOD, 4, 16, 48, s) == ERR_SHAPE
    assert lib.qgemm_mxfp4_act(GOOD, GOOD, GOOD, GOOD, 0, 16, 64, s) == OK
    assert lib.qgemm_fp8_act(GOOD, GOOD, None, GOOD, GOOD, 4, 16, 64, s) == ERR_NULL
    assert lib.qgemm_fp8_act(GOOD, GOOD, GOOD, GOOD, None, 4, 16, 64, s) == ERR_NULL
    assert lib.qgemm_fp8_act(GOOD, GOOD, GOOD, GOOD, GOOD, 4, 16, 40, s) == ERR_SHAPE
    assert lib.qgemm_fp8_act(GOOD, GOOD, GOOD, GOOD, GOOD, 0, 16, 64, s) == OK


def test_grouped_prepack_bytes(lib):
    # codes as for the per-column format, 256-aligned, then 4 bytes per column,
    # K tile and metadata entry (1 entry per tile for group_k % 128 == 0,
    # 2 for 64, else 4)
    codes_w4 = 4096 * 4096 // 2
    assert lib.qgemm_prepack_grouped_bytes(5, 4096, 4096, 128) == codes_w4 + 4096 * 32 * 4
    assert lib.qgemm_prepack_grouped_bytes(5, 4096, 4096, 4096) == codes_w4 + 4096 * 32 * 4
    assert lib.qgemm_prepack_grouped_bytes(5, 4096, 4096, 64) == codes_w4 + 4096 * 32 * 8
    assert lib.qgemm_prepack_grouped_bytes(6, 4096, 4096, 32) == 4096 * 4096 + 4096 * 32 * 16
    assert lib.qgemm_prepack_grouped_bytes(6, 4096, 4096, 96) == 4096 * 4096 + 4096 * 32 * 16
    # 9 column groups x 2 K tiles: codes 9*2*2048 = 36864 (256-aligned), metadata 9*2*16*4
    assert lib.qgemm_prepack_grouped_bytes(6, 160, 130, 32) == 36864 + 9 * 2 * 16 * 16
    assert lib.qgemm_prepack_grouped_bytes(5, 4096, 4096, 48) == ERR_SHAPE   # group_k % 32
    assert lib.qgemm_prepack_grouped_bytes(5, 4100, 4096, 128) == ERR_SHAPE  # K % 32
    assert lib.qgemm_prepack_grouped_bytes(5, 4096, 4096, 0) == ERR_SHAPE
    assert lib.qgemm_prepack_grouped_bytes(1, 4096, 4096, 128) == ERR_FORMAT
    assert lib.qgemm_prepack_grouped_bytes(5, 0, 16, 128) == 0


def test_grouped_argument_errors_need_no_device(lib):
    s = P(0)
    pg = lib.qgemm_prepack_grouped
    assert pg(1, GOOD, GOOD, None, 128, 1, GOOD, 128, 16, s) == ERR_FORMAT
    assert pg(5, GOOD, None, None, 128, 1, GOOD, 128, 16, s) == ERR_NULL    # scales required
    assert pg(5, GOOD, GOOD, None, 128, 0, GOOD, 128, 16, s) == ERR_SHAPE   # group_n >= 1
    assert pg(5, GOOD, GOOD, None, 100, 1, GOOD, 128, 16, s) == ERR_SHAPE
    assert pg(6, GOOD, GOOD, ODD, 128, 1, GOOD, 128, 16, s) == ERR_ALIGN
    assert pg(6, None, None, None, 128, 1, GOOD, 0, 16, s) == OK            # nothing to pack
    for fn in (lib.qgemm_w4a16_grouped, lib.qgemm_w8a16_grouped):
        assert fn(None, GOOD, GOOD, 4, 16, 128, 128, s) == ERR_NULL
        assert fn(GOOD, GOOD, GOOD, 4, 16, 120, 128, s) == ERR_SHAPE       # K % 32
        assert fn(GOOD, GOOD, GOOD, 4, 16, 128, 48, s) == ERR_SHAPE        # group_k % 32
        assert fn(GOOD, ODD, GOOD, 4, 16, 128, 128, s) == ERR_ALIGN
        assert fn(GOOD, GOOD, GOOD, 0, 16, 128, 128, s) == OK              # empty: no-op


def test_binding_refuses_to_run_without_the_library(monkeypatch, tmp_path):
    monkeypatch.setattr(qg, "_lib", None)
    monkeypatch.setattr(qg, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        qg.lib()


def test_arch_check_rejects_other_architectures(lib, monkeypatch):
    """QGEMM_ERR_ARCH: a valid call on a device that is not gfx950 returns the
    status before anything is launched (the architecture name is injected)."""
    s = P(0)
    monkeypatch.setenv("QGEMM_ARCH_OVERRIDE", "gfx942")
    assert lib.qgemm_w8a16(GOOD, GOOD, GOOD, GOOD, 4, 16, 32, s) == ERR_ARCH
    assert lib.qgemm_w4a16(GOOD, GOOD, GOOD, GOOD, 4, 16, 32, s) == ERR_ARCH
    assert lib.qgemm_mxfp4(GOOD, GOOD, GOOD, GOOD, 4, 16, 64, s) == ERR_ARCH
    assert lib.qgemm_fp8(GOOD, GOOD, GOOD, GOOD, GOOD, 4, 16, 64, s) == ERR_ARCH
    assert lib.qgemm_nvfp4(GOOD, GOOD, GOOD, GOOD, 4, 16, 64, s) == ERR_ARCH
    assert lib.qgemm_w8a16_grouped(GOOD, GOOD, GOOD, 4, 16, 128, 128, s) == ERR_ARCH
    assert lib.qgemm_prepack(2, GOOD, None, GOOD, 32, 32, s) == ERR_ARCH
    assert lib.qgemm_quantize_mxfp4(GOOD, 4, 32, GOOD, GOOD, s) == ERR_ARCH
    assert lib.qgemm_quantize_fp8(GOOD, 16, GOOD, GOOD, s) == ERR_ARCH
    assert lib.qgemm_fp8_act(GOOD, GOOD, GOOD, GOOD, GOOD, 4, 16, 64, s) == ERR_ARCH
    # argument errors still come first, and empty calls stay no-ops
    assert lib.qgemm_w8a16(None, GOOD, GOOD, GOOD, 4, 16, 32, s) == ERR_NULL
    assert lib.qgemm_w8a16(GOOD, GOOD, GOOD, GOOD, 0, 16, 32, s) == OK
    monkeypatch.setenv("QGEMM_ARCH_OVERRIDE", "gfx90a")
    assert lib.qgemm_w8a16(GOOD, GOOD, GOOD, GOOD, 4, 16, 32, s) == ERR_ARCH


def test_fp8_act_noalloc_argument_errors_need_no_device(lib):
    s = P(0)
    fn = lib.qgemm_fp8_act_noalloc
    assert fn(GOOD, GOOD, None, GOOD, 4, 16, 64, s) == ERR_NULL
    assert fn(GOOD, ODD, GOOD, GOOD, 4, 16, 64, s) == ERR_ALIGN
    assert fn(GOOD, GOOD, GOOD, GOOD, 4, 16, 40, s) == ERR_SHAPE
    assert fn(GOOD, GOOD, GOOD, GOOD, 0, 16, 64, s) == OK
    # M * K past the fixed scratch (16 Mi elements) is refused on the host
    limit = qg.FP8_ACT_NOALLOC_MAX_ELEMS
    assert limit == 16 * 1024 * 1024
    assert fn(GOOD, GOOD, GOOD, GOOD, limit // 8192 + 1, 16, 8192, s) == ERR_TOO_LARGE
    assert fn(GOOD, GOOD, GOOD, GOOD, 1, 16, limit + 16, s) == ERR_TOO_LARGE
