"""GPU parity at the small-M kernel's pipeline boundaries.

Each wave of a workgroup takes the K tiles wave, wave + NW, ... and keeps
two of them in flight.  A steady loop runs while every tile it computes and
every tile it reloads exists; the last at most three tiles of a wave go
through a guarded loop, and slots past the end load through an empty
buffer.  The K tile counts below put each wave on both sides of those
boundaries: fewer tiles than slots (some waves own none), exactly the slots,
one round short of and just past the steady loop's condition, for four waves
(fewer than 16 tiles) and eight, with K a multiple of the tile or cut inside
the last tile, and with one row (activations loaded into registers) and 16
(staged through LDS).  N = 40 leaves a ragged last column group.
"""

import numpy as np
import pytest
import torch

import oracle
import qgemm_workloads as wl
import bit_quantized_gemm_qgemm_amd as qg

pytestmark = pytest.mark.gpu

# K tiles: four waves below 16 tiles (steady loop from 13), eight from 16
# (steady loop for some waves from 25, for all from 32)
TILE_COUNTS = [1, 3, 4, 5, 12, 13, 16, 24, 25, 26, 32, 33, 41]
N = 40


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


def check(y, y_ref, bound, what):
    ok = oracle.within_tolerance(host(y), y_ref, bound)
    if not ok.all():
        i, j = np.argwhere(~ok)[0]
        raise AssertionError(f"{what}: {int((~ok).sum())} of {ok.size} outside tolerance; "
                             f"first at {(i, j)}")


def k_values(tile, step):
    """K for each tile count: a whole number of tiles, and cut `step` short."""
    out = []
    for kt in TILE_COUNTS:
        out.append(kt * tile)
        if kt * tile - step > 0:
            out.append(kt * tile - step)
    return out


@pytest.mark.parametrize("m", [1, 16])
@pytest.mark.parametrize("k", k_values(128, 40))
def test_w8a16_pipeline(m, k):
    case_id("w8a16 pipeline", m, k, N)
    x, w, s = wl.w8a16(m, k, N, seed=k + m)
    y_ref, bound = oracle.gemm_w8a16(x, w, s)
    y = qg.qgemm_w8a16(dev(x), qg.qgemm_prepack("w8a16", dev(w), k, N), dev(s), N)
    check(y, y_ref, bound, f"w8a16 {m}x{k}x{N}")


@pytest.mark.parametrize("m", [1, 16])
@pytest.mark.parametrize("k", k_values(128, 40))
def test_w4a16_pipeline(m, k):
    case_id("w4a16 pipeline", m, k, N)
    x, packed, s = wl.w4a16(m, k, N, seed=k + m)
    y_ref, bound = oracle.gemm_w4a16(x, packed, s)
    y = qg.qgemm_w4a16(dev(x), qg.qgemm_prepack("w4a16", dev(packed), k, N), dev(s), N)
    check(y, y_ref, bound, f"w4a16 {m}x{k}x{N}")


@pytest.mark.parametrize("m", [1, 16])
@pytest.mark.parametrize("k", k_values(128, 48))
def test_fp8_pipeline(m, k):
    case_id("fp8 pipeline", m, k, N)
    a, b = wl.fp8_operands(m, N, k, seed=k + m)
    qa, sa = oracle.fp8_quantize(a)
    qb, sb = oracle.fp8_quantize(b)
    c_ref, bound = oracle.gemm_fp8(qa, qb, sa, sb)
    sa_d = torch.tensor([sa], dtype=torch.float32, device="cuda")
    sb_d = torch.tensor([sb], dtype=torch.float32, device="cuda")
    c = qg.qgemm_fp8(dev(qa), qg.qgemm_prepack("fp8", dev(qb), k, N), sa_d, sb_d, N)
    check(c, c_ref, bound, f"fp8 {m}x{N}x{k}")


@pytest.mark.parametrize("m", [1, 16])
@pytest.mark.parametrize("k", k_values(256, 96))
def test_mxfp4_pipeline(m, k):
    """Cut tiles also exercise the A scales past K: the bytes after a row's
    last block belong to the next row and must not reach the product."""
    case_id("mxfp4 pipeline", m, k, N)
    a, w = wl.mxfp4_operands(m, N, k, seed=k + m)
    ac, ae = oracle.mxfp4_quantize(a)
    wc, we = oracle.mxfp4_quantize(w)
    c_ref, bound = oracle.gemm_mxfp4(ac, ae, wc, we)
    wp = qg.qgemm_prepack("mxfp4", dev(wc), k, N, w_scales=dev(we))
    check(qg.qgemm_mxfp4(dev(ac), dev(ae), wp, N), c_ref, bound, f"mxfp4 {m}x{N}x{k}")


@pytest.mark.parametrize("k", [96, 1568, 4192])
def test_mxfp4_nan_scale_after_last_block(k):
    """Row r's A-scale bytes are followed by row r + 1's.  Give every row past
    the first the NaN scale (0xFF) on its first block: a kernel that took
    those bytes as the scales of row 0's blocks past K would spoil row 0.
    (K = 4192: 17 tiles, eight waves, activations staged.)"""
    m = 16
    case_id("mxfp4 NaN scale after the last block", m, k, N)
    a, w = wl.mxfp4_operands(m, N, k, seed=k)
    ac, ae = oracle.mxfp4_quantize(a)
    wc, we = oracle.mxfp4_quantize(w)
    ae = ae.copy()
    ae[1:, 0] = 0xFF
    c_ref, bound = oracle.gemm_mxfp4(ac[:1], ae[:1], wc, we)
    wp = qg.qgemm_prepack("mxfp4", dev(wc), k, N, w_scales=dev(we))
    c = qg.qgemm_mxfp4(dev(ac), dev(ae), wp, N)
    check(c[:1], c_ref, bound, f"mxfp4 {m}x{N}x{k} row 0")


@pytest.mark.parametrize("m", [1, 16])
@pytest.mark.parametrize("n", [4112, 10000, 12304, 16400])
def test_mxfp4_column_groups_per_workgroup(m, n):
    """The W scale bytes of four consecutive column groups share a word, and
    the words of eight groups form a band.  N gives 2 (4112), 3 (10000) and 4
    (12304, 16400) groups per workgroup (three straddle quads and bands),
    each with a last workgroup of fewer groups; K = 1056 cuts the last tile."""
    k = 1056
    case_id("mxfp4 scale words per quad", m, n, k)
    a, w = wl.mxfp4_operands(m, n, k, seed=n + m)
    ac, ae = oracle.mxfp4_quantize(a)
    wc, we = oracle.mxfp4_quantize(w)
    c_ref, bound = oracle.gemm_mxfp4(ac, ae, wc, we)
    wp = qg.qgemm_prepack("mxfp4", dev(wc), k, n, w_scales=dev(we))
    check(qg.qgemm_mxfp4(dev(ac), dev(ae), wp, n), c_ref, bound, f"mxfp4 {m}x{n}x{k}")


@pytest.mark.parametrize("m", [1, 9, 16])
@pytest.mark.parametrize("n,k", [(4112, 2064), (8216, 4096)])
def test_fp8_launch_shapes(m, n, k):
    """FP8 launch shapes at one slab with many column groups: up to eight
    rows one group per workgroup (eight waves), 9 .. 16 rows four waves
    loading A directly (17 or 32 K tiles: the steady loop and a cut last
    tile; N leaves a last workgroup of one group)."""
    case_id("fp8 launch shapes", m, n, k)
    a, b = wl.fp8_operands(m, n, k, seed=k + n + m)
    qa, sa = oracle.fp8_quantize(a)
    qb, sb = oracle.fp8_quantize(b)
    c_ref, bound = oracle.gemm_fp8(qa, qb, sa, sb)
    sa_d = torch.tensor([sa], dtype=torch.float32, device="cuda")
    sb_d = torch.tensor([sb], dtype=torch.float32, device="cuda")
    c = qg.qgemm_fp8(dev(qa), qg.qgemm_prepack("fp8", dev(qb), k, n), sa_d, sb_d, n)
    check(c, c_ref, bound, f"fp8 {m}x{n}x{k}")



@pytest.mark.parametrize("m,n,k", [(1, 16400, 4160), (16, 16400, 4160), (9, 20496, 4096),
                                   (16, 20496, 4096)])
def test_mxfp4_four_wave_launch(m, n, k):
    """MXFP4 with at least 16 K tiles and more than 256 workgroups of four
    column groups runs four waves loading A directly: N = 16400 gives 257
    workgroups, N = 20496 321 (each with a last workgroup of one group);
    K = 4160 cuts the last of 17 tiles, K = 4096 fills 16."""
    case_id("mxfp4 four-wave launch", m, n, k)
    a, w = wl.mxfp4_operands(m, n, k, seed=k + n + m)
    ac, ae = oracle.mxfp4_quantize(a)
    wc, we = oracle.mxfp4_quantize(w)
    c_ref, bound = oracle.gemm_mxfp4(ac, ae, wc, we)
    wp = qg.qgemm_prepack("mxfp4", dev(wc), k, n, w_scales=dev(we))
    check(qg.qgemm_mxfp4(dev(ac), dev(ae), wp, n), c_ref, bound, f"mxfp4 {m}x{n}x{k}")


@pytest.mark.parametrize("m,k", [(1, 4160), (8, 4160), (8, 4096), (16, 4160)])
def test_w8a16_four_wave_launch(m, k):
    """INT8 weights with more than 256 workgroups of four column groups
    (N = 20496: 321, the last of one group) run four waves up to eight rows
    and eight staged waves at 16; K = 4160 cuts the last of 33 tiles."""
    n = 20496
    case_id("w8a16 four-wave launch", m, k, n)
    x, w, s = wl.w8a16(m, k, n, seed=k + n + m)
    y_ref, bound = oracle.gemm_w8a16(x, w, s)
    y = qg.qgemm_w8a16(dev(x), qg.qgemm_prepack("w8a16", dev(w), k, n), dev(s), n)
    check(y, y_ref, bound, f"w8a16 {m}x{k}x{n}")
