"""GPU parity of the small-M kernel's LDS-staged activation path.

Above eight rows, with eight waves (at least 16 K tiles), the small-M kernel
copies each activation tile into LDS with whole-row DMA reads and feeds the
matrix instructions from there.  These cases cross that path's edges against
the CPU oracle: nine rows (seven padded rows of the slab copy row M - 1), a
ragged second slab, four slabs, and a last K tile that ends inside the tile
(its chunks past K are read from outside the buffer and must land as
zeros), for every format that uses the kernel.  Bar: |Y - Y_ref| <=
1e-2 * (|X| @ |W_deq|) + 1e-3 elementwise; two calls give identical bytes.
"""

import numpy as np
import pytest
import torch

import oracle
import qgemm_workloads as wl
import bit_quantized_gemm_qgemm_amd as qg

pytestmark = pytest.mark.gpu


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


# fp16 activations: K tile 128, 16-byte chunks of 8 elements; K >= 2048 keeps
# eight waves.  2120 ends 72 elements into its last tile.
FP16_CASES = [(9, 2048, 300), (16, 2120, 130), (23, 2120, 520), (32, 4096, 64)]


@pytest.mark.parametrize("m,k,n", FP16_CASES)
def test_w4a16_staged(m, k, n):
    case_id("w4a16 staged", m, k, n)
    x, packed, s = wl.w4a16(m, k, n, seed=m + k + n)
    y_ref, bound = oracle.gemm_w4a16(x, packed, s)
    wp = qg.qgemm_prepack("w4a16", dev(packed), k, n)
    check(lambda: qg.qgemm_w4a16(dev(x), wp, dev(s), n), y_ref, bound, f"w4a16 {m}x{k}x{n}")


@pytest.mark.parametrize("m,k,n", FP16_CASES)
def test_w8a16_staged(m, k, n):
    case_id("w8a16 staged", m, k, n)
    x, w, s = wl.w8a16(m, k, n, seed=m + k + n)
    y_ref, bound = oracle.gemm_w8a16(x, w, s)
    wp = qg.qgemm_prepack("w8a16", dev(w), k, n)
    check(lambda: qg.qgemm_w8a16(dev(x), wp, dev(s), n), y_ref, bound, f"w8a16 {m}x{k}x{n}")


# group_k = 32 with K = 2144: the last tile holds 96 elements (three groups)
@pytest.mark.parametrize("fmt", ["w4a16", "w8a16"])
@pytest.mark.parametrize("m,k,n,gk", [(12, 2144, 200, 32), (24, 2048, 136, 128)])
def test_grouped_staged(fmt, m, k, n, gk):
    case_id(f"{fmt} grouped staged", m, k, n, gk)
    gen = wl.w4a16_grouped if fmt == "w4a16" else wl.w8a16_grouped
    ogemm = oracle.gemm_w4a16_grouped if fmt == "w4a16" else oracle.gemm_w8a16_grouped
    x, w, s, z = gen(m, k, n, gk, 1, zeros=True, seed=m + k + n)
    y_ref, bound = ogemm(x, w, s, z, gk, 1)
    wp = qg.qgemm_prepack_grouped(f"{fmt}_grouped", dev(w), k, n, dev(s), dev(z), gk, 1)
    fn = qg.qgemm_w4a16_grouped if fmt == "w4a16" else qg.qgemm_w8a16_grouped
    check(lambda: fn(dev(x), wp, n, gk), y_ref, bound, f"{fmt} grouped {m}x{k}x{n}")


@pytest.mark.parametrize("m,k,n", [(10, 2128, 150), (30, 2048, 64)])
def test_nvfp4_staged(m, k, n):
    case_id("nvfp4 staged", m, k, n)
    x, codes, scales, g = wl.nvfp4_weight(m, k, n, seed=m + k + n)
    y_ref, bound = oracle.gemm_nvfp4(x, codes, scales, g)
    wp = qg.qgemm_prepack("nvfp4", dev(codes), k, n, w_scales=dev(scales))
    gs = torch.tensor([g], dtype=torch.float32, device="cuda")
    check(lambda: qg.qgemm_nvfp4(dev(x), wp, gs, n), y_ref, bound, f"nvfp4 {m}x{k}x{n}")


# e4m3 activations: 128-byte rows per K tile, chunks of 16 elements; 2128
# ends 80 elements into its last tile.  M = 40 and 100 take four slabs.
@pytest.mark.parametrize("m,n,k", [(9, 200, 2048), (16, 130, 2128), (24, 64, 2128),
                                   (40, 300, 2048), (100, 96, 2128)])
def test_fp8_staged(m, n, k):
    case_id("fp8 staged", m, n, k)
    a, b = wl.fp8_operands(m, n, k, seed=m + n + k)
    qa, sa = oracle.fp8_quantize(a)
    qb, sb = oracle.fp8_quantize(b)
    c_ref, bound = oracle.gemm_fp8(qa, qb, sa, sb)
    bp = qg.qgemm_prepack("fp8", dev(qb), k, n)
    sa_d = torch.tensor([sa], dtype=torch.float32, device="cuda")
    sb_d = torch.tensor([sb], dtype=torch.float32, device="cuda")
    check(lambda: qg.qgemm_fp8(dev(qa), bp, sa_d, sb_d, n), c_ref, bound, f"fp8 {m}x{n}x{k}")


# E2M1 activations: K tile 256 (128 bytes per row), chunks of 32 elements;
# K >= 4096 keeps eight waves, 4192 ends 96 elements into its last tile
@pytest.mark.parametrize("m,n,k", [(9, 130, 4096), (16, 64, 4192), (24, 200, 4192),
                                   (40, 64, 4096), (100, 136, 4192)])
def test_mxfp4_staged(m, n, k):
    case_id("mxfp4 staged", m, n, k)
    a, w = wl.mxfp4_operands(m, n, k, seed=m + n + k)
    ac, ae = oracle.mxfp4_quantize(a)
    wc, we = oracle.mxfp4_quantize(w)
    c_ref, bound = oracle.gemm_mxfp4(ac, ae, wc, we)
    wp = qg.qgemm_prepack("mxfp4", dev(wc), k, n, w_scales=dev(we))
    check(lambda: qg.qgemm_mxfp4(dev(ac), dev(ae), wp, n), c_ref, bound, f"mxfp4 {m}x{n}x{k}")
