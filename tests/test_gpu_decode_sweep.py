"""GPU parity over a seeded sweep of shapes through the small-M kernel.

The hand-picked decode cases cover each edge once.  Here a fixed, seeded
draw of shapes crosses the small-M kernel's launch choices in combination
for every format it serves (weight-only M up to 255, FP8 up to 512, MXFP4 up
to 256): one to sixteen rows (one slab, activations loaded directly, or
staged above eight rows with up to four column groups), two slabs, four
(e4m3 / E2M1 activations above 32 rows), one and several row blocks
(several: four waves per workgroup and the XCD-aware workgroup mapping with
padded column blocks), short K (four waves) against long K (eight), K tails
inside the last tile, fp16 rows that are not 16-byte aligned (K % 8 != 0,
the element-wise path), and ragged N.  Every output is checked against the
oracle with its bound, and each call is repeated for determinism.
"""

import numpy as np
import pytest
import torch

import oracle
import qgemm_workloads as wl
import bit_quantized_gemm_qgemm_amd as qg

pytestmark = pytest.mark.gpu


def _shapes(seed, count, m_range, n_range, k_values):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        m = int(rng.integers(*m_range))
        n = int(rng.integers(*n_range))
        k = int(rng.choice(k_values))
        out.append((m, n, k))
    return out


# fp16 activations: K tiles of 128 (16 tiles from K = 2048 on); K % 8 != 0
# takes the element-wise path.  Weight-only M up to 255 stays on this kernel
# (the tiled kernel needs M >= 256 and enough tiles).
FP16_K = [24, 136, 1000, 1030, 2056, 2120, 3002, 4104]
W4_SWEEP = _shapes(201, 10, (1, 129), (1, 700), FP16_K) + _shapes(202, 2, (129, 256), (1, 300), FP16_K)
W8_SWEEP = _shapes(203, 10, (1, 129), (1, 700), FP16_K + [1001, 2051]) + \
    _shapes(204, 2, (129, 256), (1, 300), FP16_K)
# e4m3: K % 16 == 0, tiles of 128; E2M1: K % 32 == 0, tiles of 256
# (the small-M kernel takes FP8 up to M = 512 and MXFP4 up to M = 256 at these N)
FP8_SWEEP = _shapes(205, 10, (1, 129), (1, 700), [16, 272, 1040, 2064, 2128, 4112]) + \
    _shapes(210, 4, (129, 513), (1, 700), [16, 272, 2064, 2128])
MX_SWEEP = _shapes(206, 10, (1, 129), (1, 700), [32, 288, 1056, 4128, 4352]) + \
    _shapes(211, 3, (129, 257), (1, 700), [288, 4128, 4352])
NV_SWEEP = _shapes(207, 8, (1, 129), (1, 700), [16, 272, 1040, 2064, 2128])
# grouped: K and the group a multiple of 32
GROUPED_SWEEP = [(m, n, k, int(g)) for (m, n, k), g in zip(
    _shapes(208, 10, (1, 129), (1, 500), [64, 288, 1056, 2080, 2144]),
    np.random.default_rng(209).choice([32, 64, 128], size=10))]


@pytest.fixture(scope="module", autouse=True)
def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    qg.lib()   # fails loudly if the library is not built
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


@pytest.mark.parametrize("m,n,k", W4_SWEEP)
def test_w4a16_decode_sweep(m, n, k):
    case_id("w4a16 decode sweep", m, n, k)
    x, packed, s = wl.w4a16(m, k, n, seed=5 * m + 3 * n + k)
    y_ref, bound = oracle.gemm_w4a16(x, packed, s)
    wp = qg.qgemm_prepack("w4a16", dev(packed), k, n)
    check(lambda: qg.qgemm_w4a16(dev(x), wp, dev(s), n), y_ref, bound, f"w4a16 {m}x{k}x{n}")


@pytest.mark.parametrize("m,n,k", W8_SWEEP)
def test_w8a16_decode_sweep(m, n, k):
    case_id("w8a16 decode sweep", m, n, k)
    x, w, s = wl.w8a16(m, k, n, seed=5 * m + 3 * n + k)
    y_ref, bound = oracle.gemm_w8a16(x, w, s)
    wp = qg.qgemm_prepack("w8a16", dev(w), k, n)
    check(lambda: qg.qgemm_w8a16(dev(x), wp, dev(s), n), y_ref, bound, f"w8a16 {m}x{k}x{n}")


@pytest.mark.parametrize("m,n,k", FP8_SWEEP)
def test_fp8_decode_sweep(m, n, k):
    case_id("fp8 decode sweep", m, n, k)
    a, b = wl.fp8_operands(m, n, k, seed=5 * m + 3 * n + k)
    qa, sa = oracle.fp8_quantize(a)
    qb, sb = oracle.fp8_quantize(b)
    c_ref, bound = oracle.gemm_fp8(qa, qb, sa, sb)
    bp = qg.qgemm_prepack("fp8", dev(qb), k, n)
    sa_d = torch.tensor([sa], dtype=torch.float32, device="cuda")
    sb_d = torch.tensor([sb], dtype=torch.float32, device="cuda")
    check(lambda: qg.qgemm_fp8(dev(qa), bp, sa_d, sb_d, n), c_ref, bound, f"fp8 {m}x{n}x{k}")


@pytest.mark.parametrize("m,n,k", MX_SWEEP)
def test_mxfp4_decode_sweep(m, n, k):
    case_id("mxfp4 decode sweep", m, n, k)
    a, w = wl.mxfp4_operands(m, n, k, seed=5 * m + 3 * n + k)
    ac, ae = oracle.mxfp4_quantize(a)
    wc, we = oracle.mxfp4_quantize(w)
    c_ref, bound = oracle.gemm_mxfp4(ac, ae, wc, we)
    wp = qg.qgemm_prepack("mxfp4", dev(wc), k, n, w_scales=dev(we))
    check(lambda: qg.qgemm_mxfp4(dev(ac), dev(ae), wp, n), c_ref, bound, f"mxfp4 {m}x{n}x{k}")


@pytest.mark.parametrize("m,n,k", NV_SWEEP)
def test_nvfp4_decode_sweep(m, n, k):
    case_id("nvfp4 decode sweep", m, n, k)
    x, codes, scales, g = wl.nvfp4_weight(m, k, n, seed=5 * m + 3 * n + k)
    y_ref, bound = oracle.gemm_nvfp4(x, codes, scales, g)
    wp = qg.qgemm_prepack("nvfp4", dev(codes), k, n, w_scales=dev(scales))
    gs = torch.tensor([g], dtype=torch.float32, device="cuda")
    check(lambda: qg.qgemm_nvfp4(dev(x), wp, gs, n), y_ref, bound, f"nvfp4 {m}x{k}x{n}")


@pytest.mark.parametrize("fmt", ["w4a16", "w8a16"])
@pytest.mark.parametrize("m,n,k,gk", GROUPED_SWEEP)
def test_grouped_decode_sweep(fmt, m, n, k, gk):
    case_id(f"{fmt} grouped decode sweep", m, n, k, gk)
    gen = wl.w4a16_grouped if fmt == "w4a16" else wl.w8a16_grouped
    ogemm = oracle.gemm_w4a16_grouped if fmt == "w4a16" else oracle.gemm_w8a16_grouped
    x, w, s, z = gen(m, k, n, gk, 1, zeros=True, seed=5 * m + 3 * n + k)
    y_ref, bound = ogemm(x, w, s, z, gk, 1)
    wp = qg.qgemm_prepack_grouped(f"{fmt}_grouped", dev(w), k, n, dev(s), dev(z), gk, 1)
    fn = qg.qgemm_w4a16_grouped if fmt == "w4a16" else qg.qgemm_w8a16_grouped
    check(lambda: fn(dev(x), wp, n, gk), y_ref, bound, f"{fmt} grouped {m}x{k}x{n} g{gk}")
