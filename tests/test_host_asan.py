"""AddressSanitizer pass over the library's host-side argument checks.

Builds tests/asan_abi_check.cpp against libqgemm's host code (api.cpp built
with the sanitizer on its host pass only; the kernel objects are the normal
build) and runs it.  Every call in that program is answered on the host before
anything is launched, so no GPU is needed; the run fails on any sanitizer
report or unexpected status.
"""

import os
import shutil
import subprocess

import pytest

from conftest import ROOT

PKG = os.path.join(ROOT, "bit_quantized_gemm_qgemm_amd")
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(ROOT, "_build", "asan")
CLANG = "/opt/rocm/llvm/bin/clang++"


def run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, f"{' '.join(cmd)}\n{res.stdout}\n{res.stderr}"
    return res


@pytest.mark.skipif(not os.path.exists(CLANG) or shutil.which("hipcc") is None,
                    reason="ROCm clang toolchain not found")
def test_host_checks_are_clean_under_address_sanitizer():
    from bit_quantized_gemm_qgemm_amd import build

    build.build()   # the kernel objects under _build/ match the sources
    os.makedirs(OUT, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    api_o = os.path.join(OUT, "api_asan.o")
    run([build._hipcc(), "--offload-arch=gfx950", "-std=c++17", "-fPIC", "-O1", "-g",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
         *inc, "-x", "hip", "-c", os.path.join(CSRC, "api.cpp"), "-o", api_o])
    drv_o = os.path.join(OUT, "asan_abi_check.o")
    run([CLANG, "-std=c++17", "-O1", "-g", "-fsanitize=address", "-fno-omit-frame-pointer",
         *inc, "-c", os.path.join(ROOT, "tests", "asan_abi_check.cpp"), "-o", drv_o])
    kernels = [os.path.join(build.BUILD_DIR, os.path.splitext(s)[0] + ".o")
               for s in build.SOURCES if s != "api.cpp"]
    exe = os.path.join(OUT, "asan_abi_check")
    run([CLANG, "-fsanitize=address", drv_o, api_o, *kernels, "-L/opt/rocm/lib",
         "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=23")
    env.pop("QGEMM_ARCH_OVERRIDE", None)
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert "AddressSanitizer" not in res.stderr, res.stderr
    assert res.returncode == 0, res.stdout + res.stderr
    assert "ok (0 failures)" in res.stdout
