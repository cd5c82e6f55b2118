"""Degenerate shapes on the device, for every GEMM entry point: M = 0 or
N = 0 leave nothing to compute and must succeed with an empty result; K = 0
makes every output the empty sum, exactly 0 (on both the small-M and the
tiled dispatch); an empty tensor quantizes to no codes and the all-zero
scale rule (1.0)."""

import numpy as np
import pytest
import torch

import qgemm_workloads as wl
import bit_quantized_gemm_qgemm_amd as qg

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    qg.lib()
    return torch.device("cuda:0")


def z(shape, dtype):
    return torch.zeros(shape, dtype=dtype, device="cuda")


def empty_packed():
    return z((0,), torch.uint8)


def case_id(*a):
    print("case", *a, flush=True)


def assert_zero(t, shape):
    torch.cuda.synchronize()
    assert tuple(t.shape) == shape
    assert torch.count_nonzero(t.float()) == 0


def test_mxfp4_degenerate():
    case_id("mxfp4 degenerate")
    w = torch.from_numpy(wl.mxfp4_operands(1, 32, 64)[1]).cuda()
    wc, we = qg.qgemm_quantize_mxfp4(w)
    wp = qg.qgemm_prepack("mxfp4", wc, 64, 32, w_scales=we)
    assert qg.qgemm_mxfp4(z((0, 32), torch.uint8), z((0, 2), torch.uint8), wp, 32).shape == (0, 32)
    assert qg.qgemm_mxfp4(z((4, 32), torch.uint8), z((4, 2), torch.uint8), empty_packed(),
                          0).shape == (4, 0)
    for m, n in ((20, 24), (200, 136)):
        assert_zero(qg.qgemm_mxfp4(z((m, 0), torch.uint8), z((m, 0), torch.uint8),
                                   empty_packed(), n), (m, n))


def test_fp8_degenerate():
    case_id("fp8 degenerate")
    one = torch.ones(1, dtype=torch.float32, device="cuda")
    bp = qg.qgemm_prepack("fp8", z((64, 32), torch.uint8), 64, 32)
    assert qg.qgemm_fp8(z((0, 64), torch.uint8), bp, one, one, 32).shape == (0, 32)
    assert qg.qgemm_fp8(z((4, 64), torch.uint8), empty_packed(), one, one, 0).shape == (4, 0)
    for m, n in ((4, 24), (200, 136)):   # small-M kernel, tiled kernel
        assert_zero(qg.qgemm_fp8(z((m, 0), torch.uint8), empty_packed(), one, one, n), (m, n))


@pytest.mark.parametrize("fmt", ["w4a16_grouped", "w8a16_grouped"])
def test_grouped_degenerate(fmt):
    case_id(fmt, "degenerate")
    fn = qg.qgemm_w4a16_grouped if fmt == "w4a16_grouped" else qg.qgemm_w8a16_grouped
    gen = wl.w4a16_grouped if fmt == "w4a16_grouped" else wl.w8a16_grouped
    _, w, s, zp = gen(1, 64, 32, 32)
    wp = qg.qgemm_prepack_grouped(fmt, torch.from_numpy(w).cuda(), 64, 32,
                                  torch.from_numpy(s).cuda(), torch.from_numpy(zp).cuda(), 32)
    assert fn(z((0, 64), torch.float16), wp, 32, 32).shape == (0, 32)
    assert fn(z((4, 64), torch.float16), empty_packed(), 0, 32).shape == (4, 0)
    for m, n in ((4, 24), (300, 136)):
        assert_zero(fn(z((m, 0), torch.float16), empty_packed(), n, 32), (m, n))


def test_nvfp4_degenerate():
    case_id("nvfp4 degenerate")
    g = torch.ones(1, dtype=torch.float32, device="cuda")
    wp = qg.qgemm_prepack("nvfp4", z((32, 32), torch.uint8), 64, 32, w_scales=z((32, 4), torch.uint8))
    assert qg.qgemm_nvfp4(z((0, 64), torch.float16), wp, g, 32).shape == (0, 32)
    assert qg.qgemm_nvfp4(z((4, 64), torch.float16), empty_packed(), g, 0).shape == (4, 0)
    for m, n in ((4, 24), (300, 136)):
        assert_zero(qg.qgemm_nvfp4(z((m, 0), torch.float16), empty_packed(), g, n), (m, n))


def test_act_degenerate():
    case_id("act degenerate")
    one = torch.ones(1, dtype=torch.float32, device="cuda")
    bp = qg.qgemm_prepack("fp8", z((64, 32), torch.uint8), 64, 32)
    c, _ = qg.qgemm_fp8_act(z((0, 64), torch.float32), bp, one, 32)
    assert c.shape == (0, 32)
    for m, n in ((4, 24), (200, 136)):
        c, ws = qg.qgemm_fp8_act(z((m, 0), torch.float32), empty_packed(), one, n)
        assert_zero(c, (m, n))
        # the all-zero scale rule applies to an empty A as well
        assert ws[:4].view(torch.float32).item() == 1.0
        c, _ = qg.qgemm_mxfp4_act(z((m, 0), torch.float32), empty_packed(), n)
        assert_zero(c, (m, n))


def test_quantizers_empty():
    case_id("quantizers empty")
    codes, scale = qg.qgemm_quantize_fp8(z((0,), torch.float32))
    torch.cuda.synchronize()
    assert codes.numel() == 0 and scale.item() == 1.0
    c, e = qg.qgemm_quantize_mxfp4(z((0, 64), torch.float32))
    assert c.shape == (0, 32) and e.shape == (0, 2)


# --------------------------------------------------------------------------
# packed weights of 2^31 bytes or more: past the 32-bit buffer offsets of the
# 256 x 256 kernels, so these calls take the 128 x 128 kernel, which
# addresses with 64 bits; columns whose packed bytes sit on both sides of the
# 2^31-byte mark are checked against the oracle
# --------------------------------------------------------------------------

def random_bytes(shape, seed, lo=0, hi=256):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return torch.randint(lo, hi, shape, generator=g, device="cuda", dtype=torch.int32).to(
        torch.uint8)


def test_fp8_packed_weight_over_2gib():
    import oracle
    m, k = 256, 65536
    n = 32768 + 64           # packed B: 2^31 + 4 MiB (column group 2048 starts at 2^31)
    case_id("fp8 packed B over 2 GiB", m, n, k)
    assert qg.qgemm_prepack_bytes(4, k, n) > 1 << 31
    a = random_bytes((m, k), 21)
    b = random_bytes((k, n), 22)
    a[(a & 0x7f) == 0x7f] = 0x38          # no NaN codes
    b[(b & 0x7f) == 0x7f] = 0x30
    sa = torch.tensor([0.01], dtype=torch.float32, device="cuda")
    sb = torch.tensor([0.02], dtype=torch.float32, device="cuda")
    bp = qg.qgemm_prepack("fp8", b, k, n)
    c = qg.qgemm_fp8(a, bp, sa, sb, n)
    cols = np.array([0, 1, 32767, 32768, 32769, 32800, n - 1])
    cols_d = torch.from_numpy(cols).cuda()
    got = c[:, cols_d].float().cpu().numpy().astype(np.float64)
    qa = a.cpu().numpy()
    qb = b[:, cols_d].cpu().numpy()
    del c, bp, b
    torch.cuda.empty_cache()
    c_ref, bound = oracle.gemm_fp8(qa, qb, np.float32(0.01), np.float32(0.02))
    assert np.all(oracle.within_tolerance(got, c_ref, bound))


def test_mxfp4_packed_weight_over_2gib():
    import oracle
    m, k = 256, 65536
    n = 61696                # codes 1928 MiB, then a scale segment reaching past 2^31
    case_id("mxfp4 packed W over 2 GiB", m, n, k)
    assert qg.qgemm_prepack_bytes(3, k, n) > 1 << 31
    ac = random_bytes((m, k // 2), 31)
    ae = random_bytes((m, k // 32), 32, 120, 135)
    wc = random_bytes((n, k // 2), 33)
    we = random_bytes((n, k // 32), 34, 120, 135)
    wp = qg.qgemm_prepack("mxfp4", wc, k, n, w_scales=we)
    c = qg.qgemm_mxfp4(ac, ae, wp, n)
    # column groups from 3840 (column 61440) on keep their scales past 2^31
    cols = np.array([0, 1, 30000, 61439, 61440, 61441, n - 1])
    cols_d = torch.from_numpy(cols).cuda()
    got = c[:, cols_d].float().cpu().numpy().astype(np.float64)
    w_c, w_e = wc[cols_d].cpu().numpy(), we[cols_d].cpu().numpy()
    a_c, a_e = ac.cpu().numpy(), ae.cpu().numpy()
    del c, wp, wc, we
    torch.cuda.empty_cache()
    c_ref, bound = oracle.gemm_mxfp4(a_c, a_e, w_c, w_e)
    assert np.all(oracle.within_tolerance(got, c_ref, bound))


def _w8a16_reference_in_k_chunks(x, w, s, step=1 << 22):
    """The oracle's product and bound, summed over K chunks (both are sums
    over k, so the chunks add exactly in fp64 up to rounding)."""
    import oracle
    s_np = s.cpu().numpy()
    y = np.zeros((x.shape[0], w.shape[1]))
    bound = np.zeros_like(y)
    for k0 in range(0, x.shape[1], step):
        k1 = min(x.shape[1], k0 + step)
        yc, bc = oracle.gemm_w8a16(x[:, k0:k1].cpu().numpy(), w[k0:k1].cpu().numpy(), s_np)
        y += yc
        bound += bc
    return y, bound


def test_decode_rows_and_weight_stream_over_2gib():
    """W8A16 with M = 16, K = 2^27 - 64 and N = 16 through the small-M kernel:
    4 GiB of activations (256 MB per row) and one column group of 2 GiB
    packed weights.  A lane's activation offset counts from its workgroup's
    first row in 32 bits, so the call runs as two launches of eight rows;
    each weight tile's buffer starts at the tile, so the 2 GiB stream needs
    no offset past 2^31.  M = 1 on the same operands takes a single launch.
    Every output is checked against the oracle, accumulated over K."""
    import oracle
    m, k, n = 16, (1 << 27) - 64, 16
    case_id("w8a16 decode rows and weight stream over 2 GiB", m, k, n)
    assert qg.qgemm_dispatch_kernel("w8a16", m, n, k) == "decode_gemm_kernel"
    assert qg.qgemm_prepack_bytes(2, k, n) >= 1 << 31
    g = torch.Generator(device="cuda").manual_seed(41)
    x = torch.randn((m, k), generator=g, device="cuda", dtype=torch.float32).half()
    w = torch.randint(-127, 128, (k, n), generator=g, device="cuda", dtype=torch.int8)
    s = (torch.rand((n,), generator=g, device="cuda") * 0.008 + 0.002).half()
    wp = qg.qgemm_prepack("w8a16", w, k, n)
    y = qg.qgemm_w8a16(x, wp, s, n).float().cpu().numpy().astype(np.float64)
    y1 = qg.qgemm_w8a16(x[:1], wp, s, n).float().cpu().numpy().astype(np.float64)
    del wp
    y_ref, bound = _w8a16_reference_in_k_chunks(x, w, s)
    del x, w
    torch.cuda.empty_cache()
    assert np.all(oracle.within_tolerance(y, y_ref, bound))
    assert np.all(oracle.within_tolerance(y1, y_ref[:1], bound[:1]))


LONG_ROWS_K = 72 << 20   # 151 MB fp16 rows: 15 rows span 2.26 GB, past 2^31


def _long_rows_x(m, k, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return torch.randn((m, k), generator=g, device="cuda", dtype=torch.float32).half()


def test_grouped_decode_rows_over_2gib():
    """The grouped entry point runs activation rows longer than the small-M
    kernel's 32-bit offsets allow as row chunks too: M = 16, K = 72 Mi
    (2.4 GB of fp16 X, chunks of 15 rows and 1), N = 16, grouped INT4 with
    group 128; every output against the oracle summed over K."""
    import oracle
    m, k, n, gk = 16, LONG_ROWS_K, 16, 128
    case_id("grouped decode rows over 2 GiB", m, k, n)
    x = _long_rows_x(m, k, 43)
    w = random_bytes((k // 2, n), 44)
    g = torch.Generator(device="cuda").manual_seed(48)
    s = (torch.rand((k // gk, n), generator=g, device="cuda") * 0.015 + 0.005).half()
    z = random_bytes((k // gk, n), 45, 0, 16)
    wp = qg.qgemm_prepack_grouped("w4a16_grouped", w, k, n, s, z, gk, 1)
    y = qg.qgemm_w4a16_grouped(x, wp, n, gk).float().cpu().numpy().astype(np.float64)
    del wp
    y_ref = np.zeros((m, n))
    bound = np.zeros((m, n))
    step = 1 << 23
    for k0 in range(0, k, step):
        k1 = min(k, k0 + step)
        yc, bc = oracle.gemm_w4a16_grouped(
            x[:, k0:k1].cpu().numpy(), w[k0 // 2:k1 // 2].cpu().numpy(),
            s[k0 // gk:k1 // gk].cpu().numpy(), z[k0 // gk:k1 // gk].cpu().numpy(), gk, 1)
        y_ref += yc
        bound += bc
    del x, w, s, z
    torch.cuda.empty_cache()
    assert np.all(oracle.within_tolerance(y, y_ref, bound))


def test_nvfp4_decode_rows_over_2gib():
    """As above for NVFP4 weights (codes [N, K/2], e4m3 block scales with
    exponent field 4..10)."""
    import oracle
    m, k, n = 16, LONG_ROWS_K, 16
    case_id("nvfp4 decode rows over 2 GiB", m, k, n)
    x = _long_rows_x(m, k, 49)
    codes = random_bytes((n, k // 2), 46)
    scales = random_bytes((n, k // 16), 47, 32, 88)
    gs = torch.tensor([0.01], dtype=torch.float32, device="cuda")
    wp = qg.qgemm_prepack("nvfp4", codes, k, n, w_scales=scales)
    y = qg.qgemm_nvfp4(x, wp, gs, n).float().cpu().numpy().astype(np.float64)
    del wp
    y_ref = np.zeros((m, n))
    bound = np.zeros((m, n))
    step = 1 << 23
    for k0 in range(0, k, step):
        k1 = min(k, k0 + step)
        yc, bc = oracle.gemm_nvfp4(x[:, k0:k1].cpu().numpy(), codes[:, k0 // 2:k1 // 2].cpu().numpy(),
                                   scales[:, k0 // 16:k1 // 16].cpu().numpy(), np.float32(0.01))
        y_ref += yc
        bound += bc
    del x, codes, scales
    torch.cuda.empty_cache()
    assert np.all(oracle.within_tolerance(y, y_ref, bound))
