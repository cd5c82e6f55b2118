"""qgemm_fp8_act_noalloc: the FP8 GEMM with device-side activation
quantization that allocates nothing (its scratch is a fixed per-GPU array).

Called through the C ABI and checked against qgemm_fp8_act (the same kernels
with a caller workspace): identical output bytes, and within the tolerance of
the oracle's product of the oracle-quantized operands.  Several calls in a
row, each smaller than the last, so stale scratch contents from the previous
call would show; the largest accepted size and the first rejected one.
"""

import ctypes

import numpy as np
import pytest
import torch

import oracle
import qgemm_workloads as wl
import bit_quantized_gemm_qgemm_amd as qg

pytestmark = pytest.mark.gpu

TOO_LARGE = -8


@pytest.fixture(scope="module", autouse=True)
def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    qg.lib()
    return torch.device("cuda:0")


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def p(t):
    return ctypes.c_void_p(t.data_ptr())


def noalloc(a_d, bp, sb, n):
    m, k = a_d.shape
    out = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = qg.lib().qgemm_fp8_act_noalloc(p(a_d), p(bp), p(sb), p(out), m, n, k, stream)
    assert st == 0, qg.status_string(st)
    return out


# (M, N, K): the 256 x 256 tile path, then the small-M path, each smaller
# than the one before
CASES = [(300, 520, 4096), (64, 256, 2048), (16, 130, 1024), (3, 48, 256)]


def test_noalloc_matches_workspace_entry_point_on_calls_in_a_row():
    for m, n, k in CASES:
        print("case fp8_act_noalloc", m, n, k, flush=True)
        a, b = wl.fp8_operands(m, n, k, seed=m + n + k)
        qb, sb = oracle.fp8_quantize(b)
        bp = qg.qgemm_prepack("fp8", dev(qb), k, n)
        sb_d = torch.tensor([sb], dtype=torch.float32, device="cuda")
        a_d = dev(a)
        c = noalloc(a_d, bp, sb_d, n)
        c_ws, ws = qg.qgemm_fp8_act(a_d, bp, sb_d, n)
        torch.cuda.synchronize()
        assert torch.equal(c.view(torch.int16), c_ws.view(torch.int16)), (m, n, k)
        qa, sa = oracle.fp8_quantize(a)
        c_ref, bound = oracle.gemm_fp8(qa, qb, sa, sb)
        got = c.float().cpu().numpy().astype(np.float64)
        assert np.all(oracle.within_tolerance(got, c_ref, bound)), (m, n, k)


def test_noalloc_largest_accepted_size_then_a_small_call():
    k = 8192
    m = qg.FP8_ACT_NOALLOC_MAX_ELEMS // k          # M * K exactly at the limit
    n = 256
    print("case fp8_act_noalloc max", m, n, k, flush=True)
    g = torch.Generator(device="cuda").manual_seed(3)
    a_d = torch.randn((m, k), generator=g, device="cuda", dtype=torch.float32)
    _, b = wl.fp8_operands(1, n, k, seed=3)
    qb, sb = oracle.fp8_quantize(b)
    bp = qg.qgemm_prepack("fp8", dev(qb), k, n)
    sb_d = torch.tensor([sb], dtype=torch.float32, device="cuda")
    c = noalloc(a_d, bp, sb_d, n)
    c_ws, _ = qg.qgemm_fp8_act(a_d, bp, sb_d, n)
    assert torch.equal(c.view(torch.int16), c_ws.view(torch.int16))
    # sampled rows against the oracle (the scale is the whole tensor's)
    a = a_d.cpu().numpy()
    qa, sa = oracle.fp8_quantize(a)
    rows = np.array([0, 1, m // 2, m - 2, m - 1])
    c_ref, bound = oracle.gemm_fp8(qa[rows], qb, sa, sb)
    got = c[torch.from_numpy(rows).cuda()].float().cpu().numpy().astype(np.float64)
    assert np.all(oracle.within_tolerance(got, c_ref, bound))
    # one element more is refused before anything is enqueued
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    big = torch.empty((m + 1, k), dtype=torch.float32, device="cuda")
    out = torch.empty((m + 1, n), dtype=torch.bfloat16, device="cuda")
    assert qg.lib().qgemm_fp8_act_noalloc(p(big), p(bp), p(sb_d), p(out), m + 1, n, k,
                                          stream) == TOO_LARGE
    del big, out, a_d
    # and a small call right after the largest one
    m2, n2, k2 = 5, 64, 512
    a2, b2 = wl.fp8_operands(m2, n2, k2, seed=8)
    qb2, sb2 = oracle.fp8_quantize(b2)
    bp2 = qg.qgemm_prepack("fp8", dev(qb2), k2, n2)
    sb2_d = torch.tensor([sb2], dtype=torch.float32, device="cuda")
    a2_d = dev(a2)
    c2 = noalloc(a2_d, bp2, sb2_d, n2)
    c2_ws, _ = qg.qgemm_fp8_act(a2_d, bp2, sb2_d, n2)
    assert torch.equal(c2.view(torch.int16), c2_ws.view(torch.int16))
    qa2, sa2 = oracle.fp8_quantize(a2)
    c2_ref, bound2 = oracle.gemm_fp8(qa2, qb2, sa2, sb2)
    assert np.all(oracle.within_tolerance(c2.float().cpu().numpy().astype(np.float64), c2_ref,
                                          bound2))
