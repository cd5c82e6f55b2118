"""GPU parity of the small-M kernel with several row blocks.

When M spans more than one row block (16 rows times the slabs per
workgroup), the small-M kernel maps its linear workgroup index to (column
block, row block) so that the row blocks of one column block run on the same
XCD, and pads the column blocks to a multiple of eight (the padding
workgroups exit at once).  These cases cross that mapping's edges against the
CPU oracle for every format that uses the kernel: three to ten row blocks
with a ragged last one, column-block counts below eight and not a multiple of
eight, the weight-only shapes from M = 256 up that take this kernel because
their tile grid is small, and seven column groups per workgroup.  Launches
with several row blocks use four waves per workgroup (two workgroups per
CU), except seven-group ones whose registers would not fit twice.
Bar: |Y - Y_ref| <= 1e-2 * (|X| @ |W_deq|) + 1e-3 elementwise (the oracle's
bound); two calls give identical bytes.
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


# fp16 activations take two 16-row slabs per workgroup above 16 rows: M = 77
# is three row blocks (the last 13 rows), M = 100 four (the last 4), M = 300
# ten; N = 136 / 300 / 1000 give 9 / 19 / 63 column groups of 16 (one group
# per workgroup at these N), padded to 16 / 24 / 64 column blocks.  M = 300
# with N = 136 has two 256 x 256 tiles, too few for the tiled kernel.
FP16_CASES = [(77, 2048, 136), (100, 2120, 300), (128, 4096, 1000), (300, 2048, 136)]


@pytest.mark.parametrize("m,k,n", FP16_CASES)
def test_w4a16_row_blocks(m, k, n):
    case_id("w4a16 row blocks", m, k, n)
    x, packed, s = wl.w4a16(m, k, n, seed=3 * m + k + n)
    y_ref, bound = oracle.gemm_w4a16(x, packed, s)
    wp = qg.qgemm_prepack("w4a16", dev(packed), k, n)
    check(lambda: qg.qgemm_w4a16(dev(x), wp, dev(s), n), y_ref, bound, f"w4a16 {m}x{k}x{n}")


@pytest.mark.parametrize("m,k,n", FP16_CASES)
def test_w8a16_row_blocks(m, k, n):
    case_id("w8a16 row blocks", m, k, n)
    x, w, s = wl.w8a16(m, k, n, seed=3 * m + k + n)
    y_ref, bound = oracle.gemm_w8a16(x, w, s)
    wp = qg.qgemm_prepack("w8a16", dev(w), k, n)
    check(lambda: qg.qgemm_w8a16(dev(x), wp, dev(s), n), y_ref, bound, f"w8a16 {m}x{k}x{n}")


@pytest.mark.parametrize("fmt", ["w4a16", "w8a16"])
@pytest.mark.parametrize("m,k,n,gk", [(70, 2048, 200, 128), (97, 2144, 64, 32)])
def test_grouped_row_blocks(fmt, m, k, n, gk):
    case_id(f"{fmt} grouped row blocks", m, k, n, gk)
    gen = wl.w4a16_grouped if fmt == "w4a16" else wl.w8a16_grouped
    ogemm = oracle.gemm_w4a16_grouped if fmt == "w4a16" else oracle.gemm_w8a16_grouped
    x, w, s, z = gen(m, k, n, gk, 1, zeros=True, seed=3 * m + k + n)
    y_ref, bound = ogemm(x, w, s, z, gk, 1)
    wp = qg.qgemm_prepack_grouped(f"{fmt}_grouped", dev(w), k, n, dev(s), dev(z), gk, 1)
    fn = qg.qgemm_w4a16_grouped if fmt == "w4a16" else qg.qgemm_w8a16_grouped
    check(lambda: fn(dev(x), wp, n, gk), y_ref, bound, f"{fmt} grouped {m}x{k}x{n}")


# N = 28672 gives 1792 column groups, seven per workgroup: the widest
# register ring, with four waves per workgroup for INT4 (per-column scales
# and group 128) and eight for NVFP4 and group 64
def test_w4a16_seven_groups_row_blocks():
    m, k, n = 40, 2048, 28672
    case_id("w4a16 seven groups row blocks", m, k, n)
    x, packed, s = wl.w4a16(m, k, n, seed=11)
    y_ref, bound = oracle.gemm_w4a16(x, packed, s)
    wp = qg.qgemm_prepack("w4a16", dev(packed), k, n)
    check(lambda: qg.qgemm_w4a16(dev(x), wp, dev(s), n), y_ref, bound, f"w4a16 {m}x{k}x{n}")


@pytest.mark.parametrize("gk", [128, 64])
def test_grouped_w4a16_seven_groups_row_blocks(gk):
    m, k, n = 40, 2048, 28672
    case_id("w4a16 grouped seven groups row blocks", m, k, n, gk)
    x, w, s, z = wl.w4a16_grouped(m, k, n, gk, 1, zeros=True, seed=12)
    y_ref, bound = oracle.gemm_w4a16_grouped(x, w, s, z, gk, 1)
    wp = qg.qgemm_prepack_grouped("w4a16_grouped", dev(w), k, n, dev(s), dev(z), gk, 1)
    check(lambda: qg.qgemm_w4a16_grouped(dev(x), wp, n, gk), y_ref, bound,
          f"w4a16 grouped {m}x{k}x{n} g{gk}")


@pytest.mark.parametrize("m,k,n", [(90, 2128, 150), (128, 2048, 64), (40, 2048, 28672)])
def test_nvfp4_row_blocks(m, k, n):
    case_id("nvfp4 row blocks", m, k, n)
    x, codes, scales, g = wl.nvfp4_weight(m, k, n, seed=3 * m + k + n)
    y_ref, bound = oracle.gemm_nvfp4(x, codes, scales, g)
    wp = qg.qgemm_prepack("nvfp4", dev(codes), k, n, w_scales=dev(scales))
    gs = torch.tensor([g], dtype=torch.float32, device="cuda")
    check(lambda: qg.qgemm_nvfp4(dev(x), wp, gs, n), y_ref, bound, f"nvfp4 {m}x{k}x{n}")


# e4m3 and E2M1 activations take four slabs above 32 rows: M = 65 is two row
# blocks (the second one row), M = 128 two full ones
@pytest.mark.parametrize("m,n,k", [(65, 200, 2048), (128, 136, 2128)])
def test_fp8_row_blocks(m, n, k):
    case_id("fp8 row blocks", m, n, k)
    a, b = wl.fp8_operands(m, n, k, seed=3 * m + n + k)
    qa, sa = oracle.fp8_quantize(a)
    qb, sb = oracle.fp8_quantize(b)
    c_ref, bound = oracle.gemm_fp8(qa, qb, sa, sb)
    bp = qg.qgemm_prepack("fp8", dev(qb), k, n)
    sa_d = torch.tensor([sa], dtype=torch.float32, device="cuda")
    sb_d = torch.tensor([sb], dtype=torch.float32, device="cuda")
    check(lambda: qg.qgemm_fp8(dev(qa), bp, sa_d, sb_d, n), c_ref, bound, f"fp8 {m}x{n}x{k}")


@pytest.mark.parametrize("m,n,k", [(65, 64, 4096), (128, 300, 4192)])
def test_mxfp4_row_blocks(m, n, k):
    case_id("mxfp4 row blocks", m, n, k)
    a, w = wl.mxfp4_operands(m, n, k, seed=3 * m + n + k)
    ac, ae = oracle.mxfp4_quantize(a)
    wc, we = oracle.mxfp4_quantize(w)
    c_ref, bound = oracle.gemm_mxfp4(ac, ae, wc, we)
    wp = qg.qgemm_prepack("mxfp4", dev(wc), k, n, w_scales=dev(we))
    check(lambda: qg.qgemm_mxfp4(dev(ac), dev(ae), wp, n), c_ref, bound, f"mxfp4 {m}x{n}x{k}")
