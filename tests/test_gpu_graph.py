"""Entry points captured in a HIP graph and replayed.

A serving loop captures its GEMM calls once and replays them.  Each case
below captures one call (outputs and workspaces allocated beforehand, so the
captured call allocates nothing) and replays the graph three times; between
replays the program clears the output and writes new input values in place
with eager work of its own.  Every replay must give the same bytes as an
eager call on the same inputs: the launches read the live buffers, and no
kernel depends on memory state that a replay does not recreate (none of them
clears memory with a fill node: scratch that must start at zero is written
by the kernels themselves).
"""

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


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def case_id(*a):
    print("case", *a, flush=True)


def replay_matches_eager(call, out, refill):
    """call(): the entry point writing into `out`; refill(i): eager in-place
    rewrite of the inputs before replay i."""
    call()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for i in range(3):
        refill(i)
        call()                       # eager reference on the new inputs
        torch.cuda.synchronize()
        ref = out.clone()
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"replay {i}"


def fp16_refill(x):
    base = x.clone()
    return lambda i: x.copy_(base * (1.0 + 0.5 * i))


@pytest.mark.parametrize("fmt,m,k,n", [
    ("w8a16", 16, 4096, 1100),     # small-M kernel, one row block
    ("w4a16", 100, 2048, 700),     # several row blocks: four waves, XCD mapping
    ("w4a16", 1024, 256, 3072),    # 256 x 256 tiles (48 tiles from M = 640)
    ("w8a16", 1024, 256, 3072),
])
def test_weight_only_graph(fmt, m, k, n):
    case_id("graph", fmt, m, k, n)
    gen = wl.w4a16 if fmt == "w4a16" else wl.w8a16
    x, w, s = gen(m, k, n, seed=m + k + n)
    x, wp, s = dev(x), qg.qgemm_prepack(fmt, dev(w), k, n), dev(s)
    out = torch.empty((m, n), dtype=torch.float16, device="cuda")
    fn = qg.qgemm_w4a16 if fmt == "w4a16" else qg.qgemm_w8a16
    replay_matches_eager(lambda: fn(x, wp, s, n, out=out), out, fp16_refill(x))


def test_grouped_and_nvfp4_graph():
    m, k, n, gk = 24, 2048, 600, 64
    case_id("graph grouped", m, k, n, gk)
    x, w, s, z = wl.w4a16_grouped(m, k, n, gk, 1, zeros=True, seed=3)
    x = dev(x)
    wp = qg.qgemm_prepack_grouped("w4a16_grouped", dev(w), k, n, dev(s), dev(z), gk, 1)
    out = torch.empty((m, n), dtype=torch.float16, device="cuda")
    replay_matches_eager(lambda: qg.qgemm_w4a16_grouped(x, wp, n, gk, out=out), out,
                         fp16_refill(x))
    case_id("graph nvfp4", m, k, n)
    x, codes, scales, g = wl.nvfp4_weight(m, k, n, seed=4)
    x = dev(x)
    wp = qg.qgemm_prepack("nvfp4", dev(codes), k, n, w_scales=dev(scales))
    gs = torch.tensor([g], dtype=torch.float32, device="cuda")
    out = torch.empty((m, n), dtype=torch.float16, device="cuda")
    replay_matches_eager(lambda: qg.qgemm_nvfp4(x, wp, gs, n, out=out), out, fp16_refill(x))


@pytest.mark.parametrize("m,n,k", [(16, 1024, 2048), (512, 512, 1024)])
def test_mxfp4_graph(m, n, k):
    case_id("graph mxfp4", m, n, k)
    a, w = wl.mxfp4_operands(m, n, k, seed=m + n)
    ac, ae = qg.qgemm_quantize_mxfp4(dev(a))
    wc, we = qg.qgemm_quantize_mxfp4(dev(w))
    wp = qg.qgemm_prepack("mxfp4", wc, k, n, w_scales=we)
    out = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    codes0, scales0 = ac.clone(), ae.clone()

    def refill(i):   # rotate A's rows: new codes and scales, still valid ones
        ac.copy_(torch.roll(codes0, i + 1, 0))
        ae.copy_(torch.roll(scales0, i + 1, 0))
    replay_matches_eager(lambda: qg.qgemm_mxfp4(ac, ae, wp, n, out=out), out, refill)


@pytest.mark.parametrize("m,n,k", [(64, 1024, 2048), (1024, 1024, 512)])
def test_fp8_graph(m, n, k):
    case_id("graph fp8", m, n, k)
    a, b = wl.fp8_operands(m, n, k, seed=m + n)
    qa, sa = qg.qgemm_quantize_fp8(dev(a))
    qb, sb = qg.qgemm_quantize_fp8(dev(b))
    bp = qg.qgemm_prepack("fp8", qb, k, n)
    out = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    qa0 = qa.clone()
    replay_matches_eager(lambda: qg.qgemm_fp8(qa, bp, sa, sb, n, out=out), out,
                         lambda i: qa.copy_(torch.roll(qa0, i + 1, 0)))


@pytest.mark.parametrize("m,n,k", [(16, 1024, 2048), (300, 520, 1024)])
def test_act_graph(m, n, k):
    """The fused-quantization calls: the quantizer kernels and the GEMM in one
    graph; the workspace (and, for the allocation-free call, the library's
    fixed scratch) is rewritten by every replay before it is read."""
    case_id("graph act", m, n, k)
    a, b = wl.fp8_operands(m, n, k, seed=m + k)
    a = dev(a)
    qb, sb = qg.qgemm_quantize_fp8(dev(b))
    bp = qg.qgemm_prepack("fp8", qb, k, n)
    base = a.clone()
    refill = lambda i: a.copy_(base * (0.5 + i))   # a new per-tensor scale each time
    ws = torch.empty(max(qg.qgemm_act_workspace_bytes("fp8", m, k), 16), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    replay_matches_eager(lambda: qg.qgemm_fp8_act(a, bp, sb, n, workspace=ws, out=out), out,
                         refill)
    out2 = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    replay_matches_eager(lambda: qg.qgemm_fp8_act_noalloc(a, bp, sb, n, out2), out2, refill)
    _, wf = wl.mxfp4_operands(1, n, k, seed=5)
    wc, we = qg.qgemm_quantize_mxfp4(dev(wf))
    wp = qg.qgemm_prepack("mxfp4", wc, k, n, w_scales=we)
    wsm = torch.empty(max(qg.qgemm_act_workspace_bytes("mxfp4", m, k), 16), dtype=torch.uint8,
                      device="cuda")
    out3 = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    replay_matches_eager(lambda: qg.qgemm_mxfp4_act(a, wp, n, workspace=wsm, out=out3), out3,
                         refill)
