"""GPU parity on both sides of the dispatch rules between the small-M kernel
and the tiled kernels.

The weight-only GEMMs (per-column INT4 / INT8, grouped, NVFP4 weights) take
the 256 x 256 tiled kernel from M = 256 on once its grid of
T = ceil(M / 256) * ceil(N / 256) tiles reaches 192, or from M = 640 once
T >= 48; otherwise the small-M kernel.  FP8 and MXFP4 take the small-M
kernel up to M = 64, from 65 to 128 rows unless N is wide (FP8 N >= 24576,
MXFP4 N >= 16384: one row of 256 x 256 tiles), and above that FP8 up to
M = 512 while M * N <= 2621440, MXFP4 up to M = 256 while M * N <= 2^21;
otherwise the tiled kernels.  Each pair
of cases below sits on the two sides of one edge of a rule, so both kernels
run at the shapes where the dispatch switches.  Every output is checked against the oracle
(bar: |Y - Y_ref| <= 1e-2 * (|X| @ |W_deq|) + 1e-3 elementwise) and each
call is repeated for determinism.
"""

import numpy as np
import pytest
import torch

import oracle
import qgemm_workloads as wl
import bit_quantized_gemm_qgemm_amd as qg

pytestmark = pytest.mark.gpu

# (m, k, n): small-M kernel / tiled kernel
EDGES = [
    (256, 256, 24576),    # T = 96, M < 640: small-M kernel
    (257, 256, 24576),    # T = 192: tiles
    (639, 200, 12288),    # T = 144, M < 640: small-M kernel
    (640, 200, 12288),    # T = 144, M >= 640: tiles
    (1024, 136, 2816),    # T = 44: small-M kernel
    (1280, 136, 2560),    # T = 50, M >= 640: tiles
]


@pytest.fixture(scope="module", autouse=True)
def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    qg.lib()
    return torch.device("cuda:0")


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def case_id(*a):
    print("case", *a, flush=True)


def check(fn, y_ref, bound, what):
    y = fn()
    y2 = fn()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), f"{what}: not deterministic"
    y = host(y)
    ok = oracle.within_tolerance(y, y_ref, bound)
    if not ok.all():
        i, j = np.argwhere(~ok)[0]
        raise AssertionError(f"{what}: {int((~ok).sum())} of {ok.size} outside tolerance; "
                             f"first at {(i, j)}: got {y[i, j]!r}, want {y_ref[i, j]!r}")


@pytest.mark.parametrize("m,k,n", EDGES)
def test_w4a16_dispatch_edges(m, k, n):
    case_id("w4a16 dispatch edge", m, k, n)
    x, packed, s = wl.w4a16(m, k, n, seed=m + k + n)
    y_ref, bound = oracle.gemm_w4a16(x, packed, s)
    wp = qg.qgemm_prepack("w4a16", dev(packed), k, n)
    check(lambda: qg.qgemm_w4a16(dev(x), wp, dev(s), n), y_ref, bound, f"w4a16 {m}x{k}x{n}")


@pytest.mark.parametrize("m,k,n", EDGES)
def test_w8a16_dispatch_edges(m, k, n):
    case_id("w8a16 dispatch edge", m, k, n)
    x, w, s = wl.w8a16(m, k, n, seed=m + k + n)
    y_ref, bound = oracle.gemm_w8a16(x, w, s)
    wp = qg.qgemm_prepack("w8a16", dev(w), k, n)
    check(lambda: qg.qgemm_w8a16(dev(x), wp, dev(s), n), y_ref, bound, f"w8a16 {m}x{k}x{n}")


@pytest.mark.parametrize("m,k,n", [(256, 256, 24576), (257, 256, 24576), (639, 224, 12288),
                                   (640, 224, 12288)])
def test_grouped_dispatch_edges(m, k, n):
    case_id("w4a16 grouped dispatch edge", m, k, n)
    x, w, s, z = wl.w4a16_grouped(m, k, n, 64, 1, zeros=True, seed=m + k + n)
    y_ref, bound = oracle.gemm_w4a16_grouped(x, w, s, z, 64, 1)
    wp = qg.qgemm_prepack_grouped("w4a16_grouped", dev(w), k, n, dev(s), dev(z), 64, 1)
    check(lambda: qg.qgemm_w4a16_grouped(dev(x), wp, n, 64), y_ref, bound,
          f"w4a16 grouped {m}x{k}x{n}")


@pytest.mark.parametrize("m,k,n", [(256, 256, 24576), (257, 256, 24576), (1024, 144, 2816),
                                   (1280, 144, 2560)])
def test_nvfp4_dispatch_edges(m, k, n):
    case_id("nvfp4 dispatch edge", m, k, n)
    x, codes, scales, g = wl.nvfp4_weight(m, k, n, seed=m + k + n)
    y_ref, bound = oracle.gemm_nvfp4(x, codes, scales, g)
    wp = qg.qgemm_prepack("nvfp4", dev(codes), k, n, w_scales=dev(scales))
    gs = torch.tensor([g], dtype=torch.float32, device="cuda")
    check(lambda: qg.qgemm_nvfp4(dev(x), wp, gs, n), y_ref, bound, f"nvfp4 {m}x{k}x{n}")


# FP8: (m, n, k), small-M kernel / tiles
FP8_EDGES = [
    (512, 5120, 256),     # M * N = 2621440: small-M kernel
    (512, 5136, 256),     # M * N above: 256 x 256 tiles
    (129, 20320, 256),    # small-M kernel
    (129, 20336, 256),    # tiles
    (512, 64, 272),       # small-M kernel
    (513, 64, 272),       # M > 512: 128 x 128 tiles (N <= 128)
    (128, 24560, 256),    # 65 .. 128 rows, N < 24576: small-M kernel
    (128, 24576, 256),    # N >= 24576: one row of 256 x 256 tiles
    (64, 25000, 272),     # M <= 64: small-M kernel
    (65, 25000, 272),     # 256 x 256 tiles with 65 of their 256 rows, K tail of 16
    (100, 24600, 128),    # one 128-element K tile: 128 x 128 tiles
]


@pytest.mark.parametrize("m,n,k", FP8_EDGES)
def test_fp8_dispatch_edges(m, n, k):
    case_id("fp8 dispatch edge", m, n, k)
    a, b = wl.fp8_operands(m, n, k, seed=m + n + k)
    qa, sa = oracle.fp8_quantize(a)
    qb, sb = oracle.fp8_quantize(b)
    c_ref, bound = oracle.gemm_fp8(qa, qb, sa, sb)
    bp = qg.qgemm_prepack("fp8", dev(qb), k, n)
    sa_d = torch.tensor([sa], dtype=torch.float32, device="cuda")
    sb_d = torch.tensor([sb], dtype=torch.float32, device="cuda")
    check(lambda: qg.qgemm_fp8(dev(qa), bp, sa_d, sb_d, n), c_ref, bound, f"fp8 {m}x{n}x{k}")


# MXFP4: (m, n, k), small-M kernel / tiles
MX_EDGES = [
    (256, 8192, 512),     # M * N = 2^21: small-M kernel
    (256, 8208, 512),     # M * N above: 256 x 256 tiles
    (256, 200, 640),      # small-M kernel
    (257, 200, 640),      # M > 256: 256 x 256 tiles
    (200, 10485, 288),    # small-M kernel (M * N = 2097000)
    (200, 10500, 288),    # tiles: K = 288 is not a multiple of 128, the 128 x 128 kernel
    (128, 16368, 512),    # 65 .. 128 rows, N < 16384: small-M kernel
    (128, 16384, 512),    # N >= 16384: one row of 256 x 256 tiles
    (64, 17000, 640),     # M <= 64: small-M kernel
    (65, 17000, 640),     # 256 x 256 tiles with 65 of their 256 rows
    (100, 16400, 288),    # K = 288: 128 x 128 tiles
]


@pytest.mark.parametrize("m,n,k", MX_EDGES)
def test_mxfp4_dispatch_edges(m, n, k):
    case_id("mxfp4 dispatch edge", m, n, k)
    a, w = wl.mxfp4_operands(m, n, k, seed=m + n + k)
    ac, ae = oracle.mxfp4_quantize(a)
    wc, we = oracle.mxfp4_quantize(w)
    c_ref, bound = oracle.gemm_mxfp4(ac, ae, wc, we)
    wp = qg.qgemm_prepack("mxfp4", dev(wc), k, n, w_scales=dev(we))
    check(lambda: qg.qgemm_mxfp4(dev(ac), dev(ae), wp, n), c_ref, bound, f"mxfp4 {m}x{n}x{k}")
