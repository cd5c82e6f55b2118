"""GPU parity over a seeded sweep of shapes through the 256 x 256 kernels.

The hand-picked cases elsewhere cover each edge once; here a fixed,
seeded draw of shapes crosses them in combination (ragged M and N against
every K tail the kernels distinguish), so the buffer-resource bounds, the
per-step offsets and the schedules of the large-tile paths are exercised on
many tile grids.  Every output is checked against the oracle (same
tolerance as the parity tests), and each call is repeated for determinism.
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


# MXFP4: M > 256 (the small-M kernel's limit at these N) and N > 128 take the
# 256 x 256 kernel when K % 128 == 0 (K >= 512); other multiples of 32 take
# the 128 x 128 kernel
MX_SWEEP = _shapes(101, 10, (257, 900), (129, 700), [512, 640, 768, 896, 1152, 1408]) + \
    _shapes(102, 4, (257, 720), (129, 520), [544, 608, 800])
# FP8: M > 512 (the small-M kernel's limit at these N), N > 128 and at least
# two 128-element K tiles; K % 16 == 0
FP8_SWEEP = _shapes(103, 12, (513, 1100), (129, 700), [256, 272, 400, 528, 1024, 1040, 1296])
# weight-only tile path: M >= 640 with 64 to 81 tiles of 256 x 256; K % 8 == 0
WO_SWEEP = _shapes(104, 3, (1793, 2100), (1793, 2100), [136, 264, 392])


@pytest.fixture(scope="module", autouse=True)
def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    qg.lib()   # fails loudly if the library is not built
    return torch.device("cuda:0")


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def check(y, y_ref, bound, what):
    ok = oracle.within_tolerance(y, y_ref, bound)
    if not ok.all():
        i, j = np.argwhere(~ok)[0]
        raise AssertionError(f"{what}: {int((~ok).sum())} of {ok.size} outside tolerance; "
                             f"first at {(i, j)}: got {y[i, j]!r}, want {y_ref[i, j]!r}")


def case_id(*a):
    print("case", *a, flush=True)


@pytest.mark.parametrize("m,n,k", MX_SWEEP)
def test_mxfp4_sweep(m, n, k):
    case_id("mxfp4 sweep", m, n, k)
    a, w = wl.mxfp4_operands(m, n, k, seed=7 * m + 5 * n + k)
    ac, ae = oracle.mxfp4_quantize(a)
    wc, we = oracle.mxfp4_quantize(w)
    c_ref, bound = oracle.gemm_mxfp4(ac, ae, wc, we)
    wp = qg.qgemm_prepack("mxfp4", dev(wc), k, n, w_scales=dev(we))
    c = qg.qgemm_mxfp4(dev(ac), dev(ae), wp, n)
    check(host(c), c_ref, bound, f"mxfp4 {m}x{n}x{k}")
    c2 = qg.qgemm_mxfp4(dev(ac), dev(ae), wp, n)
    assert torch.equal(c.view(torch.int16), c2.view(torch.int16))


@pytest.mark.parametrize("m,n,k", FP8_SWEEP)
def test_fp8_sweep(m, n, k):
    case_id("fp8 sweep", m, n, k)
    a, b = wl.fp8_operands(m, n, k, seed=7 * m + 5 * n + k)
    qa, sa = oracle.fp8_quantize(a)
    qb, sb = oracle.fp8_quantize(b)
    c_ref, bound = oracle.gemm_fp8(qa, qb, sa, sb)
    bp = qg.qgemm_prepack("fp8", dev(qb), k, n)
    sa_d = torch.tensor([sa], dtype=torch.float32, device="cuda")
    sb_d = torch.tensor([sb], dtype=torch.float32, device="cuda")
    c = qg.qgemm_fp8(dev(qa), bp, sa_d, sb_d, n)
    check(host(c), c_ref, bound, f"fp8 {m}x{n}x{k}")
    c2 = qg.qgemm_fp8(dev(qa), bp, sa_d, sb_d, n)
    assert torch.equal(c.view(torch.int16), c2.view(torch.int16))


@pytest.mark.parametrize("m,n,k", WO_SWEEP)
def test_w4a16_tile_sweep(m, n, k):
    case_id("w4a16 tile sweep", m, n, k)
    x, packed, s = wl.w4a16(m, k, n, seed=7 * m + 5 * n + k)
    y_ref, bound = oracle.gemm_w4a16(x, packed, s)
    wp = qg.qgemm_prepack("w4a16", dev(packed), k, n)
    y = qg.qgemm_w4a16(dev(x), wp, dev(s), n)
    check(host(y), y_ref, bound, f"w4a16 {m}x{k}x{n}")


@pytest.mark.parametrize("m,n,k", WO_SWEEP)
def test_w8a16_tile_sweep(m, n, k):
    case_id("w8a16 tile sweep", m, n, k)
    x, w, s = wl.w8a16(m, k, n, seed=7 * m + 5 * n + k)
    y_ref, bound = oracle.gemm_w8a16(x, w, s)
    wp = qg.qgemm_prepack("w8a16", dev(w), k, n)
    y = qg.qgemm_w8a16(dev(x), wp, dev(s), n)
    check(host(y), y_ref, bound, f"w8a16 {m}x{k}x{n}")
