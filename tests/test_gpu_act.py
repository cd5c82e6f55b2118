"""GPU parity of the entry points that quantize fp32 activations on the device
and run the GEMM in the same call (qgemm_mxfp4_act, qgemm_fp8_act).

Bars: the workspace holds the oracle quantizer's codes, E8M0 bytes and FP8
scale bit-exactly; the output equals the two-call sequence (quantize entry
point, then GEMM entry point) bit for bit; and it is within
1e-2 * (|A_deq| @ |W_deq|) + 1e-3 of the oracle.
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


def case_id(*a):
    print("case", *a, flush=True)


def bits(t):
    return t.view(torch.int16).cpu()


@pytest.mark.parametrize("m,n,k", [(16, 300, 512), (64, 96, 256), (300, 260, 640), (1, 16, 32)])
def test_mxfp4_act(m, n, k):
    case_id("mxfp4 act", m, n, k)
    a, w = wl.mxfp4_operands(m, n, k, seed=m + n + k)
    wc, we = oracle.mxfp4_quantize(w)
    wp = qg.qgemm_prepack("mxfp4", dev(wc), k, n, w_scales=dev(we))
    c, ws = qg.qgemm_mxfp4_act(dev(a), wp, n)
    ac, ae = oracle.mxfp4_quantize(a)
    wsn = ws.cpu().numpy()
    off = -(-m * k // 2 // 16) * 16
    assert np.array_equal(wsn[:m * k // 2].reshape(m, k // 2), ac)
    assert np.array_equal(wsn[off:off + m * k // 32].reshape(m, k // 32), ae)
    qa, qe = qg.qgemm_quantize_mxfp4(dev(a))
    c2 = qg.qgemm_mxfp4(qa, qe, wp, n)
    assert torch.equal(bits(c), bits(c2))
    c_ref, bound = oracle.gemm_mxfp4(ac, ae, wc, we)
    assert oracle.within_tolerance(c.float().cpu().numpy(), c_ref, bound).all()


@pytest.mark.parametrize("m,n,k", [(16, 300, 512), (1, 64, 128), (200, 272, 384), (600, 272, 384),
                                   (17, 16, 16)])
def test_fp8_act(m, n, k):
    case_id("fp8 act", m, n, k)
    a, b = wl.fp8_operands(m, n, k, seed=m + n + k)
    qb, sb = oracle.fp8_quantize(b)
    bp = qg.qgemm_prepack("fp8", dev(qb), k, n)
    sb_d = torch.tensor([sb], dtype=torch.float32, device="cuda")
    c, ws = qg.qgemm_fp8_act(dev(a), bp, sb_d, n)
    qa, sa = oracle.fp8_quantize(a)
    wsn = ws.cpu().numpy()
    off = -(-m * k // 16) * 16
    assert np.array_equal(wsn[:m * k].reshape(m, k), qa)
    assert wsn[off:off + 4].view(np.float32)[0] == np.float32(sa)
    qa_d, sa_d = qg.qgemm_quantize_fp8(dev(a))
    c2 = qg.qgemm_fp8(qa_d, bp, sa_d, sb_d, n)
    assert torch.equal(bits(c), bits(c2))
    c_ref, bound = oracle.gemm_fp8(qa, qb, sa, sb)
    assert oracle.within_tolerance(c.float().cpu().numpy(), c_ref, bound).all()


def test_fp8_act_decode_full_size_sampled():
    """The FP8 decode shape (M = 16, K = N = 8192) with A quantized in the call."""
    m, n, k = 16, 8192, 8192
    case_id("fp8 act full", m, n, k)
    a, b = wl.fp8_operands(m, n, k)
    qb, sb = oracle.fp8_quantize(b)
    bp = qg.qgemm_prepack("fp8", dev(qb), k, n)
    c, ws = qg.qgemm_fp8_act(dev(a), bp, torch.tensor([sb], dtype=torch.float32, device="cuda"), n)
    qa, sa = oracle.fp8_quantize(a)
    assert np.array_equal(ws.cpu().numpy()[:m * k].reshape(m, k), qa)
    cols = np.unique(np.concatenate([np.random.default_rng(3).integers(0, n, 96), [0, n - 1]]))
    c_ref, bound = oracle.gemm_fp8(qa, qb[:, cols], sa, sb)
    assert oracle.within_tolerance(c.float().cpu().numpy()[:, cols], c_ref, bound).all()
