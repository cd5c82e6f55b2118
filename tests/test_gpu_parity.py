"""GPU parity: every libqgemm entry point against the CPU oracle.

Bars:
  * bit-exact for integer and byte results: MXFP4 / e4m3fn quantizer codes,
    E8M0 bytes and the FP8 scale, and one-hot read-backs of the dequantized
    weights through the real GEMM kernels (a single-term fp32 sum is exact, so
    the stored output equals the output-rounded dequantized weight);
  * elsewhere |Y - Y_ref| <= 1e-2 * (|X| @ |W_deq|) + 1e-3 elementwise, with
    Y_ref the oracle's fp64 product of the dequantized operands;
  * determinism: two calls give identical bytes.

Small cases span several tiles and ragged tails; the full-size workloads are
checked on sampled outputs (the oracle computes those from the sampled rows
and columns only), in the launch configuration the benchmark times.
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
    qg.lib()   # fails loudly if the library is not built
    return torch.device("cuda:0")


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def assert_within(y, y_ref, bound, what):
    ok = oracle.within_tolerance(y, y_ref, bound)
    if not ok.all():
        bad = np.argwhere(~ok)
        i, j = bad[0]
        raise AssertionError(
            f"{what}: {len(bad)} of {ok.size} outside tolerance; first at {(i, j)}: "
            f"got {y[i, j]!r}, want {y_ref[i, j]!r}, tol {oracle.tolerance(bound)[i, j]!r}")


def case_id(*a):
    print("case", *a, flush=True)


# --------------------------------------------------------------------------
# W4A16
# --------------------------------------------------------------------------

W4_CASES = [
    (16, 1024, 1024),   # the small W4A16 workload, whole
    (1, 256, 48),
    (5, 200, 33),       # K not a multiple of the 128-wide K tile, ragged N
    (3, 130, 17),       # K % 8 != 0: rows of X are not 16-byte aligned
    (16, 384, 100),
    (40, 512, 64),      # M > 16: several 16-row slabs
    (17, 128, 16),
    (8, 2048, 700),
    (16, 256, 16400),   # eight column groups per workgroup, ragged last workgroup
    (6, 384, 9000),     # four groups per workgroup (M in 5..8)
    (256, 1024, 272),   # M >= 256 with few 256 x 256 tiles: the small-M kernel, slabs
    (300, 1000, 520),   # ragged M, K tail inside the last 128-wide tile
    (513, 136, 384),    # seventeen 32-row slab pairs
    (260, 100, 300),    # K % 8 != 0 at large M: element-wise activation loads
    (32, 2048, 16400),  # two 16-row slabs per workgroup, seven column groups
    (64, 1024, 1000),   # four slabs per workgroup
    (100, 768, 3000),   # four slabs, two workgroup rows, ragged last slab
    (255, 256, 600),    # four workgroup rows of four slabs
]


@pytest.mark.parametrize("m,k,n", W4_CASES)
def test_w4a16_matches_oracle(m, k, n):
    case_id("w4a16", m, k, n)
    x, packed, s = wl.w4a16(m, k, n, seed=m * 1000 + k + n)
    y_ref, bound = oracle.gemm_w4a16(x, packed, s)
    wp = qg.qgemm_prepack("w4a16", dev(packed), k, n)
    y = qg.qgemm_w4a16(dev(x), wp, dev(s), n)
    assert_within(host(y), y_ref, bound, f"w4a16 {m}x{k}x{n}")
    y2 = qg.qgemm_w4a16(dev(x), wp, dev(s), n)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


@pytest.mark.parametrize("k,n", [(1024, 1024), (200, 33)])
def test_w4a16_one_hot_reads_back_dequantized_weights(k, n):
    """X = rows of the identity: Y[m, :] = fp16(W_deq[k_m, :]) exactly."""
    case_id("w4a16 one-hot", k, n)
    _, packed, s = wl.w4a16(1, k, n, seed=7)
    s = (s.astype(np.float32) * np.where(np.arange(n) % 3 == 0, -1, 1)).astype(np.float16)
    wdeq = oracle.round_fp16(oracle.dequant_w4(packed, s))
    wp = qg.qgemm_prepack("w4a16", dev(packed), k, n)
    for k0 in range(0, k, 16):
        rows = np.arange(k0, min(k, k0 + 16))
        x = np.zeros((len(rows), k), np.float16)
        x[np.arange(len(rows)), rows] = 1
        y = host(qg.qgemm_w4a16(dev(x), wp, dev(s), n))
        assert np.array_equal(y, wdeq[rows]), f"rows {rows[0]}..{rows[-1]}"


@pytest.mark.parametrize("m", [1, 8, 16, 48])
def test_w4a16_decode_full_size_sampled(m):
    k, n = 8192, 28672
    case_id("w4a16 decode full", m, k, n)
    x, packed, s = wl.w4a16(max(m, 16), k, n)
    x = x[:m]
    wp = qg.qgemm_prepack("w4a16", dev(packed), k, n)
    y = host(qg.qgemm_w4a16(dev(x), wp, dev(s), n))
    cols = np.unique(np.concatenate([np.random.default_rng(m).integers(0, n, 96), [0, n - 1]]))
    y_ref, bound = oracle.gemm_w4a16(x, packed[:, cols], s[cols])
    assert_within(y[:, cols], y_ref, bound, f"w4a16 full M={m}")


# --------------------------------------------------------------------------
# W8A16
# --------------------------------------------------------------------------

W8_CASES = [
    (4, 4096, 11008),
    (1, 128, 16),
    (7, 333, 50),       # K % 8 != 0
    (16, 1000, 129),    # K % 128 != 0
    (33, 256, 64),      # M > 16
    (2, 64, 1),
    (9, 200, 9000),     # four groups, short K, ragged N
    (16, 520, 2100),
    (256, 2048, 300),   # M >= 256 with few 256 x 256 tiles: the small-M kernel, slabs
    (300, 1000, 520),   # ragged M, N and K
    (260, 64, 1000),    # one K tile
    (257, 333, 200),    # K % 8 != 0 at large M: element-wise activation loads
    (32, 512, 640),     # two 16-row slabs per workgroup
    (129, 640, 2100),   # four slabs, three workgroup rows, ragged
    (64, 4096, 520),    # four slabs, long K
]


@pytest.mark.parametrize("m,k,n", W8_CASES)
def test_w8a16_matches_oracle(m, k, n):
    case_id("w8a16", m, k, n)
    x, w, s = wl.w8a16(m, k, n, seed=m * 1000 + k + n)
    y_ref, bound = oracle.gemm_w8a16(x, w, s)
    wp = qg.qgemm_prepack("w8a16", dev(w), k, n)
    y = qg.qgemm_w8a16(dev(x), wp, dev(s), n)
    assert_within(host(y), y_ref, bound, f"w8a16 {m}x{k}x{n}")
    y2 = qg.qgemm_w8a16(dev(x), wp, dev(s), n)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


def test_w8a16_page_test_distribution():
    """The W8A16 page's own test shape and distribution (w down to -128,
    scales from N(0,1) * 0.01, so negative and tiny scales)."""
    case_id("w8a16 page test")
    x, w, s = wl.w8a16_page_test(32, 128, 256)
    y_ref, bound = oracle.gemm_w8a16(x, w, s)
    wp = qg.qgemm_prepack("w8a16", dev(w), 128, 256)
    y = host(qg.qgemm_w8a16(dev(x), wp, dev(s), 256))
    assert_within(y, y_ref, bound, "w8a16 page test")


def test_w8a16_one_hot_full_byte_range():
    k, n = 256, 48
    case_id("w8a16 one-hot", k, n)
    w = ((np.arange(k)[:, None] + 37 * np.arange(n)[None, :]) % 256 - 128).astype(np.int8)
    s = np.random.default_rng(3).uniform(-0.02, 0.02, n).astype(np.float16)
    wdeq = oracle.round_fp16(oracle.dequant_w8(w, s))
    wp = qg.qgemm_prepack("w8a16", dev(w), k, n)
    for k0 in range(0, k, 16):
        x = np.zeros((16, k), np.float16)
        x[np.arange(16), k0 + np.arange(16)] = 1
        y = host(qg.qgemm_w8a16(dev(x), wp, dev(s), n))
        assert np.array_equal(y, wdeq[k0:k0 + 16])


@pytest.mark.parametrize("m", [1, 4, 16, 64])
def test_w8a16_decode_full_size_sampled(m):
    k, n = 4096, 11008
    case_id("w8a16 decode full", m, k, n)
    x, w, s = wl.w8a16(max(m, 16), k, n)
    x = x[:m]
    wp = qg.qgemm_prepack("w8a16", dev(w), k, n)
    y = host(qg.qgemm_w8a16(dev(x), wp, dev(s), n))
    cols = np.unique(np.concatenate([np.random.default_rng(m).integers(0, n, 128), [0, n - 1]]))
    y_ref, bound = oracle.gemm_w8a16(x, w[:, cols], s[cols])
    assert_within(y[:, cols], y_ref, bound, f"w8a16 full M={m}")


@pytest.mark.parametrize("fmt", ["w4a16", "w8a16"])
def test_weight_only_one_hot_through_large_tiles(fmt):
    """X = the identity (M = K = 2048, N = 2080: 8 x 9 tiles of 256 x 256, the
    tiled kernel): Y = fp16(W_deq) exactly, every weight of every tile and K
    step."""
    k, n = 2048, 2080
    case_id(f"{fmt} one-hot large tiles", k, n)
    rng = np.random.default_rng(11)
    s = (rng.uniform(0.002, 0.02, n) * np.where(np.arange(n) % 3 == 0, -1, 1)).astype(np.float16)
    if fmt == "w4a16":
        w = rng.integers(0, 256, size=(k // 2, n)).astype(np.uint8)
        wdeq = oracle.round_fp16(oracle.dequant_w4(w, s))
        fn = qg.qgemm_w4a16
    else:
        w = ((np.arange(k)[:, None] + 37 * np.arange(n)[None, :]) % 256 - 128).astype(np.int8)
        wdeq = oracle.round_fp16(oracle.dequant_w8(w, s))
        fn = qg.qgemm_w8a16
    wp = qg.qgemm_prepack(fmt, dev(w), k, n)
    x = np.eye(k, dtype=np.float16)
    y = host(fn(dev(x), wp, dev(s), n))
    assert np.array_equal(y, wdeq)


# M >= 640 with at least 48 tiles of 256 x 256: the tiled kernel (K tail, short K, one K tile).
TILED_CASES = [(2048, 1000, 2100), (2304, 136, 2048), (2050, 64, 2304)]


@pytest.mark.parametrize("fmt", ["w4a16", "w8a16"])
@pytest.mark.parametrize("m,k,n", TILED_CASES)
def test_weight_only_tiled_sampled(fmt, m, k, n):
    case_id(f"{fmt} tiled", m, k, n)
    gen = wl.w4a16 if fmt == "w4a16" else wl.w8a16
    x, w, s = gen(m, k, n, seed=m + k + n)
    wp = qg.qgemm_prepack(fmt, dev(w), k, n)
    fn = qg.qgemm_w4a16 if fmt == "w4a16" else qg.qgemm_w8a16
    y = host(fn(dev(x), wp, dev(s), n))
    rng = np.random.default_rng(k)
    rows = np.unique(np.concatenate([rng.integers(0, m, 64), [0, 255, 256, m - 1]]))
    cols = np.unique(np.concatenate([rng.integers(0, n, 64), [0, 255, 256, n - 1]]))
    gemm = oracle.gemm_w4a16 if fmt == "w4a16" else oracle.gemm_w8a16
    y_ref, bound = gemm(x[rows], w[:, cols], s[cols])
    assert_within(y[np.ix_(rows, cols)], y_ref, bound, f"{fmt} tiled sampled")


@pytest.mark.parametrize("fmt", ["w4a16", "w8a16"])
def test_weight_only_square_full_size_sampled(fmt):
    """M = N = K = 4096 (the W8A16 page's fused-versus-explicit comparison
    shape) on sampled rows and columns."""
    m = k = n = 4096
    case_id(f"{fmt} square full", m, k, n)
    gen = wl.w4a16 if fmt == "w4a16" else wl.w8a16
    x, w, s = gen(m, k, n)
    wp = qg.qgemm_prepack(fmt, dev(w), k, n)
    fn = qg.qgemm_w4a16 if fmt == "w4a16" else qg.qgemm_w8a16
    y = host(fn(dev(x), wp, dev(s), n))
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([rng.integers(0, m, 48), [0, m - 1]]))
    cols = np.unique(np.concatenate([rng.integers(0, n, 48), [0, n - 1]]))
    gemm = oracle.gemm_w4a16 if fmt == "w4a16" else oracle.gemm_w8a16
    y_ref, bound = gemm(x[rows], w[:, cols], s[cols])
    assert_within(y[np.ix_(rows, cols)], y_ref, bound, f"{fmt} square sampled")


def test_weight_only_empty_and_zero_k():
    case_id("weight-only empty")
    x = torch.zeros((4, 0), dtype=torch.float16, device="cuda")
    for fmt, fn in (("w8a16", qg.qgemm_w8a16), ("w4a16", qg.qgemm_w4a16)):
        wp = torch.zeros(16, dtype=torch.uint8, device="cuda")
        s = torch.ones(20, dtype=torch.float16, device="cuda")
        y = fn(x, wp, s, 20)
        torch.cuda.synchronize()
        assert torch.count_nonzero(y) == 0
    # M = 0: a no-op that leaves nothing to compare but must not fail
    x0 = torch.zeros((0, 64), dtype=torch.float16, device="cuda")
    wp = qg.qgemm_prepack("w8a16", torch.zeros((64, 8), dtype=torch.int8, device="cuda"), 64, 8)
    assert qg.qgemm_w8a16(x0, wp, torch.ones(8, dtype=torch.float16, device="cuda"), 8).shape == (0, 8)


def test_weight_only_rejects_odd_k_for_w4():
    x = torch.zeros((2, 7), dtype=torch.float16, device="cuda")
    with pytest.raises(qg.QgemmError):
        qg.qgemm_w4a16(x, torch.zeros(1024, dtype=torch.uint8, device="cuda"),
                       torch.ones(16, dtype=torch.float16, device="cuda"), 16)


# --------------------------------------------------------------------------
# MXFP4
# --------------------------------------------------------------------------

def varied(rng, rows, k):
    x = rng.standard_normal((rows, k)).astype(np.float32) * np.float32(0.5)
    mags = np.ldexp(1.0, rng.integers(-12, 12, size=(rows, k // 32))).astype(np.float32)
    x = (x.reshape(rows, k // 32, 32) * mags[..., None]).reshape(rows, k)
    x[0, :32] = 0.0                                  # an all-zero block
    x[min(1, rows - 1), 32:64] = np.float32(6.0) * np.float32(0.25)  # ties at the grid
    return x


@pytest.mark.parametrize("rows,k", [(3, 64), (37, 256), (128, 8192), (1, 32)])
def test_mxfp4_quantizer_bit_exact(rows, k):
    case_id("mxfp4 quantize", rows, k)
    x = varied(np.random.default_rng(rows + k), rows, k)
    want_c, want_e = oracle.mxfp4_quantize(x)
    c, e = qg.qgemm_quantize_mxfp4(dev(x))
    assert np.array_equal(c.cpu().numpy(), want_c)
    assert np.array_equal(e.cpu().numpy(), want_e)


def test_mxfp4_quantizer_ties_and_edges_bit_exact():
    case_id("mxfp4 quantize ties")
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    vals = []
    for m in mids:
        m32 = np.float32(m)
        vals += [m32, np.nextafter(m32, np.float32(0)), np.nextafter(m32, np.float32(9))]
    vals = np.array(vals, np.float32)
    rows = []
    for e in (-20, -3, 0, 5, 30):
        blk = np.zeros(32, np.float32)
        blk[0] = np.float32(6.0 * 2.0 ** e)
        blk[1:1 + len(vals)] = vals * np.float32(2.0 ** e)
        blk[-1] = -blk[2]
        rows.append(blk)
        edge = np.float32(6.0 * 2.0 ** e)
        for v in (np.nextafter(edge, np.float32(np.inf)), np.nextafter(edge, np.float32(0))):
            b2 = blk.copy()
            b2[0] = v
            rows.append(b2)
    x = np.stack(rows).astype(np.float32)
    want_c, want_e = oracle.mxfp4_quantize(x)
    c, e = qg.qgemm_quantize_mxfp4(dev(x))
    assert np.array_equal(c.cpu().numpy(), want_c)
    assert np.array_equal(e.cpu().numpy(), want_e)


MX_CASES = [
    (64, 64, 256),
    (300, 70, 96),      # 128 x 128 tiles: ragged M, N, K (K not a multiple of the 256-wide step)
    (130, 70, 96),      # the same ragged N and K through the small-M kernel above 128 rows
    (1, 16, 32),
    (257, 129, 544),
    (260, 256, 1024),
    (256, 256, 1024),   # small-M kernel: M = 256 with M * N <= 2^21
    (16, 300, 2048),
    (300, 260, 640),    # 256 x 256 tiles: ragged M and N, K a multiple of 128
    (512, 512, 1024),
    (129, 16300, 384),  # M * N > 2^21: 256 x 256 tiles; K = 384, a half 256-wide step at the end
    (129, 1000, 384),   # the same K through the small-M kernel
    (257, 384, 1280),   # 256 x 256 tiles, several pipeline iterations
    (300, 136, 896),    # last 128-wide step all padding; 9 column tiles
    (100, 520, 800),    # small-M kernel: four slabs, two workgroup rows, K = 3.125 tiles
    (33, 136, 288),     # four slabs, one row of them ragged; K = 1.125 tiles
    (128, 2100, 256),
    (200, 600, 4128),   # small-M kernel above 128 rows: four row blocks of 64, eight waves' K
    (1024, 2048, 512),  # 4 x 8 tiles of 256 x 256: the tile count is a multiple of 8,
                        # so the XCD-remapped walk and its 4-row groups run
    (1280, 1792, 768),  # 5 x 7 = 35 tiles (plain walk), ragged group of tile rows
    (2048, 1024, 1024), # 8 x 4 tiles: remapped walk, two 4-row groups
    (512, 768, 2048),   # 6 tiles (plain walk), eight K steps
    (2304, 2560, 2560), # 90 tiles, ten K steps: the copy ring wraps its four stages
    (4352, 4096, 2048), # 272 tiles: more than one per CU, remapped walk
]


@pytest.mark.parametrize("m,n,k", MX_CASES)
def test_mxfp4_gemm_matches_oracle(m, n, k):
    case_id("mxfp4 gemm", m, n, k)
    a, w = wl.mxfp4_operands(m, n, k, seed=m + n + k)
    ac, ae = oracle.mxfp4_quantize(a)
    wc, we = oracle.mxfp4_quantize(w)
    c_ref, bound = oracle.gemm_mxfp4(ac, ae, wc, we)
    wp = qg.qgemm_prepack("mxfp4", dev(wc), k, n, w_scales=dev(we))
    c = qg.qgemm_mxfp4(dev(ac), dev(ae), wp, n)
    assert_within(host(c), c_ref, bound, f"mxfp4 {m}x{n}x{k}")
    c2 = qg.qgemm_mxfp4(dev(ac), dev(ae), wp, n)
    assert torch.equal(c.view(torch.int16), c2.view(torch.int16))


def test_mxfp4_one_hot_reads_back_dequantized_weights():
    """A row m holds a single 1.0 at k_m (scale 2^0): C[m, n] = W_deq[n, k_m],
    exact in bf16 (E2M1 values carry two significant bits).  M = 64 (the
    small-M kernel); N = 272 spans three groups of eight column tiles, so
    every position of a tile's scale byte is read back."""
    n, k = 272, 512
    case_id("mxfp4 one-hot", n, k)
    _, w = wl.mxfp4_operands(1, n, k, seed=5)
    wc, we = oracle.mxfp4_quantize(w)
    wdeq = oracle.mxfp4_dequant(wc, we)
    wp = qg.qgemm_prepack("mxfp4", dev(wc), k, n, w_scales=dev(we))
    for k0 in range(0, k, 64):
        m = 64
        codes = np.zeros((m, k), np.uint8)
        codes[np.arange(m), k0 + np.arange(m)] = 0b0010        # +1.0
        ac = oracle.pack_nibbles_last_axis(codes)
        ae = np.full((m, k // 32), 127, np.uint8)
        c = host(qg.qgemm_mxfp4(dev(ac), dev(ae), wp, n))
        assert np.array_equal(c, wdeq[:, k0:k0 + m].T)


@pytest.mark.parametrize("m,n,k", [(300, 272, 512), (512, 768, 2048)])
def test_mxfp4_one_hot_through_large_tiles(m, n, k):
    """One-hot read-back through the 256 x 256 kernel (M > 256, N > 128): every
    (row tile, column tile, K step, scale byte) mapping is hit, bit-exact."""
    case_id("mxfp4 one-hot large tiles", m, n, k)
    _, w = wl.mxfp4_operands(1, n, k, seed=9)
    wc, we = oracle.mxfp4_quantize(w)
    wdeq = oracle.mxfp4_dequant(wc, we)
    wp = qg.qgemm_prepack("mxfp4", dev(wc), k, n, w_scales=dev(we))
    ks = (np.arange(m) * 37) % k           # row i reads back column k_i of W
    codes = np.zeros((m, k), np.uint8)
    codes[np.arange(m), ks] = 0b0010        # +1.0
    ac = oracle.pack_nibbles_last_axis(codes)
    ae = np.full((m, k // 32), 127, np.uint8)
    c = host(qg.qgemm_mxfp4(dev(ac), dev(ae), wp, n))
    assert np.array_equal(c, wdeq[:, ks].T)


def test_mxfp4_scale_product_is_exponent_add_on_device():
    """One active 32-block of 1.0 * 1.0 with scales E_A, E_W gives exactly
    32 * 2^(E_A + E_W - 254) (MXFP4 page, section 2, eq. 2)."""
    case_id("mxfp4 e8m0 identity")
    rng = np.random.default_rng(9)
    m, n, k = 32, 32, 256
    ea = rng.integers(90, 165, size=m).astype(np.uint8)
    ew = rng.integers(90, 165, size=n).astype(np.uint8)
    blk = 3
    a_codes = np.zeros((m, k), np.uint8)
    a_codes[:, 32 * blk:32 * blk + 32] = 0b0010
    w_codes = np.zeros((n, k), np.uint8)
    w_codes[:, 32 * blk:32 * blk + 32] = 0b0010
    a_sc = rng.integers(100, 150, size=(m, k // 32)).astype(np.uint8)
    w_sc = rng.integers(100, 150, size=(n, k // 32)).astype(np.uint8)
    a_sc[:, blk] = ea
    w_sc[:, blk] = ew
    wp = qg.qgemm_prepack("mxfp4", dev(oracle.pack_nibbles_last_axis(w_codes)), k, n,
                          w_scales=dev(w_sc))
    c = host(qg.qgemm_mxfp4(dev(oracle.pack_nibbles_last_axis(a_codes)), dev(a_sc), wp, n))
    want = 32.0 * np.ldexp(1.0, ea[:, None].astype(np.int64) + ew[None, :] - 254)
    assert np.array_equal(c, want)


@pytest.mark.parametrize("m", [1, 16, 64])
def test_mxfp4_small_m_full_size_sampled(m):
    """K = N = 8192 at small M (the small-M kernel), on sampled columns."""
    n = k = 8192
    case_id("mxfp4 small-M full", m, n, k)
    a, w = wl.mxfp4_operands(m, n, k, seed=m)
    ac_d, ae_d = qg.qgemm_quantize_mxfp4(dev(a))
    wc_d, we_d = qg.qgemm_quantize_mxfp4(dev(w))
    wp = qg.qgemm_prepack("mxfp4", wc_d, k, n, w_scales=we_d)
    c = host(qg.qgemm_mxfp4(ac_d, ae_d, wp, n))
    cols = np.unique(np.concatenate([np.random.default_rng(m).integers(0, n, 96), [0, n - 1]]))
    ac, ae = oracle.mxfp4_quantize(a)
    wc, we = oracle.mxfp4_quantize(w[cols])
    c_ref, bound = oracle.gemm_mxfp4(ac, ae, wc, we)
    assert_within(c[:, cols], c_ref, bound, f"mxfp4 small-M full M={m}")


def tile_row_sample(m, seed, tile=256):
    """One row inside each tile row of a tile x tile output grid, at a random
    offset, plus the first and the last row."""
    rng = np.random.default_rng(seed)
    starts = np.arange(0, m, tile)
    rows = starts + rng.integers(0, tile, size=len(starts))
    return np.unique(np.concatenate([rows[rows < m], [0, m - 1]]))


def test_mxfp4_full_size_full_rows():
    """8192^3 through the 256 x 256 kernel and its XCD-remapped tile walk:
    whole output rows, one in each of the 32 tile rows, so every output tile
    is checked element by element (34 rows x 8192 columns)."""
    m = n = k = 8192
    case_id("mxfp4 full", m, n, k)
    a, w = wl.mxfp4_operands(m, n, k)
    ac_d, ae_d = qg.qgemm_quantize_mxfp4(dev(a))
    wc_d, we_d = qg.qgemm_quantize_mxfp4(dev(w))
    wp = qg.qgemm_prepack("mxfp4", wc_d, k, n, w_scales=we_d)
    c = qg.qgemm_mxfp4(ac_d, ae_d, wp, n)
    rows = tile_row_sample(m, 1)
    got = host(c[torch.from_numpy(rows).cuda()])
    del c, wp
    ac, ae = oracle.mxfp4_quantize(a[rows])
    wc = np.empty((n, k // 2), np.uint8)
    we = np.empty((n, k // 32), np.uint8)
    for r0 in range(0, n, 1024):                 # the oracle quantizes W in row chunks
        wc[r0:r0 + 1024], we[r0:r0 + 1024] = oracle.mxfp4_quantize(w[r0:r0 + 1024])
    # the device quantizer's bytes equal the oracle's on these A rows and all of W
    assert np.array_equal(ac_d[torch.from_numpy(rows).cuda()].cpu().numpy(), ac)
    assert np.array_equal(wc_d.cpu().numpy(), wc) and np.array_equal(we_d.cpu().numpy(), we)
    c_ref, bound = oracle.gemm_mxfp4(ac, ae, wc, we)
    assert_within(got, c_ref, bound, "mxfp4 8192^3 full rows")


# --------------------------------------------------------------------------
# FP8
# --------------------------------------------------------------------------

@pytest.mark.parametrize("shape", [(64, 48), (1000,), (8192, 16), (3, 5)])
def test_fp8_quantizer_bit_exact(shape):
    case_id("fp8 quantize", shape)
    rng = np.random.default_rng(sum(shape))
    x = (rng.standard_normal(shape) * np.ldexp(1.0, rng.integers(-8, 8, shape))).astype(np.float32)
    want_c, want_s = oracle.fp8_quantize(x)
    c, s = qg.qgemm_quantize_fp8(dev(x))
    assert np.array_equal(c.cpu().numpy(), want_c)
    assert s.cpu().numpy()[0] == want_s


def test_fp8_quantizer_zero_tensor():
    c, s = qg.qgemm_quantize_fp8(torch.zeros(100, dtype=torch.float32, device="cuda"))
    assert s.item() == 1.0 and torch.count_nonzero(c) == 0


FP8_CASES = [
    (16, 64, 128),      # small-M path
    (1, 48, 256),
    (7, 130, 96),
    (600, 72, 160),     # 128 x 128 tiles, ragged
    (200, 72, 160),     # the same through the small-M kernel above 128 rows
    (768, 256, 512),
    (17, 16, 16),
    (560, 260, 528),    # 256 x 256 tiles with a 16-wide K tail
    (300, 260, 528),    # the same K tail through the small-M kernel
    (512, 5200, 1024),  # M * N > 2.6e6: 256 x 256 tiles
    (512, 5120, 1024),  # M * N = 2621440: the small-M kernel's largest grid, eight row blocks
    (129, 20400, 256),  # M * N > 2.6e6 from M = 129: tiles
    (640, 300, 384),    # 256 x 256 tiles, six 64-wide steps
    (560, 200, 2064),   # 256 x 256 tiles, K tail of 16 in the last step
    (136, 200, 2064),   # the same K tail through the small-M kernel
    (32, 256, 512),     # small-M kernel, two 16-row slabs per workgroup
    (64, 1024, 2048),   # four slabs
    (100, 512, 384),    # four slabs, two workgroup rows, ragged
    (128, 2048, 256),
    (1024, 2048, 512),  # 4 x 8 tiles of 256 x 256: the XCD-remapped walk
    (2048, 1024, 1024), # 8 x 4 tiles: remapped walk, two 4-row groups
    (1200, 1800, 528),  # 5 x 8 = 40 tiles, remapped, ragged last tile row and column
]


@pytest.mark.parametrize("m,n,k", FP8_CASES)
def test_fp8_gemm_matches_oracle(m, n, k):
    case_id("fp8 gemm", m, n, k)
    a, b = wl.fp8_operands(m, n, k, seed=m + n + k)
    qa, sa = oracle.fp8_quantize(a)
    qb, sb = oracle.fp8_quantize(b)
    c_ref, bound = oracle.gemm_fp8(qa, qb, sa, sb)
    bp = qg.qgemm_prepack("fp8", dev(qb), k, n)
    sa_d = torch.tensor([sa], dtype=torch.float32, device="cuda")
    sb_d = torch.tensor([sb], dtype=torch.float32, device="cuda")
    c = qg.qgemm_fp8(dev(qa), bp, sa_d, sb_d, n)
    assert_within(host(c), c_ref, bound, f"fp8 {m}x{n}x{k}")
    c2 = qg.qgemm_fp8(dev(qa), bp, sa_d, sb_d, n)
    assert torch.equal(c.view(torch.int16), c2.view(torch.int16))


@pytest.mark.parametrize("m", [16, 64])
def test_fp8_one_hot_reads_back_codes(m):
    """A = one-hot 1.0 rows, unit scales: C[i, n] = e4m3 value of B[k_i, n]."""
    n, k = 40, 256
    case_id("fp8 one-hot", m)
    b = np.random.default_rng(4).integers(0, 256, size=(k, n)).astype(np.uint8)
    b[(b & 0x7f) == 0x7f] = 0x3c                     # no NaN codes
    bdeq = oracle.e4m3fn_decode(b)
    bp = qg.qgemm_prepack("fp8", dev(b), k, n)
    one = torch.ones(1, dtype=torch.float32, device="cuda")
    for k0 in range(0, k, m):
        a = np.zeros((m, k), np.uint8)
        a[np.arange(m), k0 + np.arange(m)] = 0x38    # e4m3 1.0
        c = host(qg.qgemm_fp8(dev(a), bp, one, one, n))
        assert np.array_equal(c, oracle.round_bf16(bdeq[k0:k0 + m]))


def test_fp8_one_hot_through_large_tiles():
    """One-hot read-back through the 256 x 256 path (M > 512, N > 128), bit-exact:
    pins the 32 x 32 accumulator layout and the K order of both operands."""
    m, n, k = 600, 272, 384
    case_id("fp8 one-hot large tiles", m, n, k)
    b = np.random.default_rng(6).integers(0, 256, size=(k, n)).astype(np.uint8)
    b[(b & 0x7f) == 0x7f] = 0x3c                     # no NaN codes
    bdeq = oracle.e4m3fn_decode(b)
    bp = qg.qgemm_prepack("fp8", dev(b), k, n)
    one = torch.ones(1, dtype=torch.float32, device="cuda")
    ks = (np.arange(m) * 37) % k
    a = np.zeros((m, k), np.uint8)
    a[np.arange(m), ks] = 0x38                       # e4m3 1.0
    c = host(qg.qgemm_fp8(dev(a), bp, one, one, n))
    assert np.array_equal(c, oracle.round_bf16(bdeq[ks]))


@pytest.mark.parametrize("m", [16, 64])
def test_fp8_full_size_sampled(m):
    n = k = 8192
    case_id("fp8 full", m, n, k)
    a, b = wl.fp8_operands(m, n, k)
    qa_d, sa_d = qg.qgemm_quantize_fp8(dev(a))
    qb_d, sb_d = qg.qgemm_quantize_fp8(dev(b))
    bp = qg.qgemm_prepack("fp8", qb_d, k, n)
    c = qg.qgemm_fp8(qa_d, bp, sa_d, sb_d, n)
    qa, sa = oracle.fp8_quantize(a)
    qb, sb = oracle.fp8_quantize(b)
    assert sa_d.item() == sa and sb_d.item() == sb
    rows, cols = wl.sample_indices(m, n, 256)
    ur, uc = np.unique(rows), np.unique(cols)
    assert np.array_equal(qa_d[torch.from_numpy(ur)].cpu().numpy(), qa[ur])
    c_ref, bound = oracle.gemm_fp8(qa[ur], qb[:, uc], sa, sb)
    ri = np.searchsorted(ur, rows)
    ci = np.searchsorted(uc, cols)
    got = host(c[torch.from_numpy(rows), torch.from_numpy(cols)])
    assert np.all(oracle.within_tolerance(got, c_ref[ri, ci], bound[ri, ci]))


def test_fp8_full_size_full_rows():
    """8192^3 through the 256 x 256 kernel and its XCD-remapped tile walk:
    whole output rows, one in each of the 32 tile rows (34 rows x 8192)."""
    m = n = k = 8192
    case_id("fp8 full rows", m, n, k)
    a, b = wl.fp8_operands(m, n, k)
    qa_d, sa_d = qg.qgemm_quantize_fp8(dev(a))
    qb_d, sb_d = qg.qgemm_quantize_fp8(dev(b))
    bp = qg.qgemm_prepack("fp8", qb_d, k, n)
    c = qg.qgemm_fp8(qa_d, bp, sa_d, sb_d, n)
    rows = tile_row_sample(m, 2)
    got = host(c[torch.from_numpy(rows).cuda()])
    del c, bp
    qa, sa = oracle.fp8_quantize(a)
    qb, sb = oracle.fp8_quantize(b)
    assert sa_d.item() == sa and sb_d.item() == sb
    assert np.array_equal(qb_d.cpu().numpy(), qb)
    c_ref, bound = oracle.gemm_fp8(qa[rows], qb, sa, sb)
    assert_within(got, c_ref, bound, "fp8 8192^3 full rows")


def test_weight_only_activations_over_2gib():
    """X of 2.7 GB (M = 40960, K = 32776 with a ragged last K tile, fp16):
    too large for the 32-bit buffer offsets of the 256 x 256 kernels, so the
    call takes a kernel that addresses with 64 bits; rows on both sides of
    the 2^31-byte mark (row 32760) match the oracle."""
    m, k = 40960, 32776
    n = 256
    case_id("w8a16 X over 2 GiB", m, k, n)
    g = torch.Generator(device="cuda").manual_seed(11)
    x = torch.randn((m, k), generator=g, device="cuda", dtype=torch.float32).half()
    _, w, s = wl.w8a16(1, k, n, seed=11)
    y = qg.qgemm_w8a16(x, qg.qgemm_prepack("w8a16", dev(w), k, n), dev(s), n)
    mark = (1 << 31) // (2 * k)
    rows = np.array([0, 1, mark - 1, mark, mark + 1, m - 1])
    xr = x[torch.from_numpy(rows).cuda()].cpu().numpy()
    y_ref, bound = oracle.gemm_w8a16(xr, w, s)
    assert_within(y[torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.float64), y_ref, bound,
                  "w8a16 X over 2 GiB")
    del x, y
    torch.cuda.empty_cache()
