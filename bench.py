"""Benchmark of the quantized GEMM hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--all]

Prints ONE JSON line for the chosen workload (default: the W8A16 decode
workload, M in {1, 4, 16}, K = 4096, N = 11008).  A step is one pass of the
whole hot path over one batch of synthetic input; for a decode workload that
is one GEMM call per listed M, for a square workload one GEMM.  Prepack and
quantization of the operands are offline and untimed; inputs are resident in
HBM before the timed region starts.

Timing: the K timed steps are captured once into a HIP graph (untimed) and
replayed once between two device synchronizations; `value` divides the work of
K steps by that wall time.  HIP events recorded on the same stream around the
replay give the average kernel duration used for the roofline figure.  Weight
buffers rotate over copies totalling >= 600 MB (more than twice the 256 MB
Infinity Cache), so each call streams its weight from HBM.  Each call's entry
in `detail` also carries `warm_us`: the same call repeated on one copy, whose
operands then stay in the caches (labelled separately; never the `value`).

The CPU baseline times the oracle (fp64 dequantize + NumPy matmul) on the host
over a bounded sample of the same workload.
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

METRIC = "weight GB/s (%HBM peak) at M≤16; TFLOPS (%MFMA peak) at M=N=K=8192"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"f16": 2500.0, "fp8": 5000.0, "fp4": 10100.0}
ROTATE_BYTES = 600e6
CALIB_BYTES = 256 * 1024 * 1024
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# GEMM kernel name -> the source file whose hash keys its traffic record
KERNEL_SOURCES = {
    "decode_gemm_kernel": "bit_quantized_gemm_qgemm_amd/csrc/decode_gemm.hip",
    "tile_gemm_kernel": "bit_quantized_gemm_qgemm_amd/csrc/tile_gemm.hip",
    "pipe256_kernel": "bit_quantized_gemm_qgemm_amd/csrc/tile_wo256.hip",
    "mxw_kernel": "bit_quantized_gemm_qgemm_amd/csrc/tile_mx256.hip",
    "f8w_kernel": "bit_quantized_gemm_qgemm_amd/csrc/tile_mx256.hip",
}

WORKLOADS = {
    # name: (format, Ms, N, K)
    "w4a16_small": ("w4a16", (16,), 1024, 1024),
    "w8a16_decode": ("w8a16", (1, 4, 16), 11008, 4096),
    "w4a16_decode": ("w4a16", (1, 8, 16), 28672, 8192),
    "mxfp4_square": ("mxfp4", (8192,), 8192, 8192),
    "fp8_square": ("fp8", (8192,), 8192, 8192),
    "fp8_decode": ("fp8", (16,), 8192, 8192),
    # the W8A16 page's fused-versus-explicit-dequant comparison shape
    "w8a16_square": ("w8a16", (4096,), 4096, 4096),
    "w4a16_square": ("w4a16", (4096,), 4096, 4096),
    # group-wise scales along K (128) with zero points, at the decode shapes
    "w4a16_g128_decode": ("w4a16_grouped", (1, 8, 16), 28672, 8192),
    "w8a16_g128_decode": ("w8a16_grouped", (1, 4, 16), 11008, 4096),
    # ... and at the large-M comparison shape (the tiled kernel)
    "w4a16_g128_square": ("w4a16_grouped", (4096,), 4096, 4096),
    "w8a16_g128_square": ("w8a16_grouped", (4096,), 4096, 4096),
    # NVFP4-style weights (e4m3 scale per 16 elements, fp32 per tensor), fp16 X
    "nvfp4_decode": ("nvfp4", (1, 8, 16), 28672, 8192),
    "nvfp4_square": ("nvfp4", (4096,), 4096, 4096),
    # MXFP4 at decode M, and batched decode (M = 32 .. 128: several 16-row
    # slabs per workgroup of the small-M kernel)
    "mxfp4_decode": ("mxfp4", (1, 16), 8192, 8192),
    "w8a16_batch": ("w8a16", (32, 64, 128), 11008, 4096),
    "w4a16_batch": ("w4a16", (32, 64, 128), 28672, 8192),
    "fp8_batch": ("fp8", (32, 64, 128), 8192, 8192),
    # fp32 activations quantized on the device inside the call, then the GEMM
    "fp8_act_decode": ("fp8_act", (16,), 8192, 8192),
    "mxfp4_act_square": ("mxfp4_act", (8192,), 8192, 8192),
}
GROUP_K = 128   # group size of the grouped workloads
SMALL_M_MAX = 128   # the largest M of the bandwidth-reported workloads
DEFAULT_WORKLOAD = "w8a16_decode"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(kernel):
    """Hash prefix of the source file that defines the GEMM kernel named in
    `kernel` (a bench label)."""
    src = next(v for k, v in KERNEL_SOURCES.items() if k in kernel)
    with open(os.path.join(ROOT, src), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


# ---------------------------------------------------------------------------
# workload set-up (device side)
# ---------------------------------------------------------------------------

class Setup:
    """Device buffers and per-call launchers of one workload."""

    def __init__(self, name):
        import torch
        import qgemm_workloads as wl
        import bit_quantized_gemm_qgemm_amd as qg

        self.name = name
        fmt, ms, n, k = WORKLOADS[name]
        self.fmt, self.ms, self.n, self.k = fmt, ms, n, k
        # workloads with M up to 128 are reported as weight GB/s against HBM
        # (their calls stream the weight through the small-M kernel); larger
        # ones as TFLOP/s
        self.kind = "decode" if max(ms) <= SMALL_M_MAX else "tile"
        self.explicit = None   # W8A16 square: the explicit dequantize-then-matmul comparison
        dev = torch.device("cuda:0")
        mmax = max(ms)
        self.calls = []        # per call: (launch(copy) -> None, alg_bytes, weight_bytes, flops)
        if fmt in ("w4a16", "w8a16"):
            gen = wl.w4a16 if fmt == "w4a16" else wl.w8a16
            x, w, s = gen(mmax, k, n)
            w_d = torch.from_numpy(w).to(dev)
            packed = qg.qgemm_prepack(fmt, w_d, k, n)
            del w_d
            s_d = torch.from_numpy(s).to(dev)
            x_d = torch.from_numpy(x).to(dev)
            w_bytes = (k * n // 2 if fmt == "w4a16" else k * n) + 2 * n
            self.copies = self._rotate(packed, w_bytes)
            fn = qg.qgemm_w4a16 if fmt == "w4a16" else qg.qgemm_w8a16
            self.dtype = "f16"
            if fmt == "w8a16" and self.kind == "tile":
                w8 = torch.from_numpy(w).to(dev)
                xm = x_d
                # the pages' unfused baseline: W_fp16 = W_int8 * s in HBM, then a GEMM
                self.explicit = lambda: torch.matmul(xm, w8.to(torch.float16) * s_d)
            for m in ms:
                xm = x_d[:m].contiguous()
                out = torch.empty((m, n), dtype=torch.float16, device=dev)
                alg = w_bytes + 2 * m * k + 2 * m * n
                self.calls.append((lambda c, xm=xm, out=out: fn(xm, self.copies[c], s_d, n, out=out),
                                   alg, w_bytes, 2 * m * n * k))
        elif fmt in ("w4a16_grouped", "w8a16_grouped"):
            w4 = fmt == "w4a16_grouped"
            gen = wl.w4a16_grouped if w4 else wl.w8a16_grouped
            x, w, s, z = gen(mmax, k, n, GROUP_K)
            packed = qg.qgemm_prepack_grouped(fmt, torch.from_numpy(w).to(dev), k, n,
                                              torch.from_numpy(s).to(dev),
                                              torch.from_numpy(z).to(dev), GROUP_K)
            x_d = torch.from_numpy(x).to(dev)
            # codes + the canonical fp16 scale and 1-byte zero point per group
            groups = -(-k // GROUP_K) * n
            w_bytes = (k * n // 2 if w4 else k * n) + 3 * groups
            self.copies = self._rotate(packed, w_bytes)
            fn = qg.qgemm_w4a16_grouped if w4 else qg.qgemm_w8a16_grouped
            self.dtype = "f16"
            for m in ms:
                xm = x_d[:m].contiguous()
                out = torch.empty((m, n), dtype=torch.float16, device=dev)
                alg = w_bytes + 2 * m * k + 2 * m * n
                self.calls.append((lambda c, xm=xm, out=out: fn(xm, self.copies[c], n, GROUP_K,
                                                                out=out),
                                   alg, w_bytes, 2 * m * n * k))
        elif fmt == "nvfp4":
            x, codes, scales, g = wl.nvfp4_weight(mmax, k, n)
            packed = qg.qgemm_prepack("nvfp4", torch.from_numpy(codes).to(dev), k, n,
                                      w_scales=torch.from_numpy(scales).to(dev))
            gs = torch.tensor([g], dtype=torch.float32, device=dev)
            x_d = torch.from_numpy(x).to(dev)
            w_bytes = k * n // 2 + k * n // 16          # codes + one e4m3 byte per 16
            self.copies = self._rotate(packed, w_bytes)
            self.dtype = "f16"
            for m in ms:
                xm = x_d[:m].contiguous()
                out = torch.empty((m, n), dtype=torch.float16, device=dev)
                alg = w_bytes + 2 * m * k + 2 * m * n
                self.calls.append((lambda c, xm=xm, out=out: qg.qgemm_nvfp4(xm, self.copies[c], gs,
                                                                            n, out=out),
                                   alg, w_bytes, 2 * m * n * k))
        elif fmt == "fp8_act":
            a, b = wl.fp8_operands(mmax, n, k)
            qb, sb = qg.qgemm_quantize_fp8(torch.from_numpy(b).to(dev))
            del b
            packed = qg.qgemm_prepack("fp8", qb, k, n)
            del qb
            a_d = torch.from_numpy(a).to(dev)
            ws = torch.empty(qg.qgemm_act_workspace_bytes("fp8", mmax, k), dtype=torch.uint8,
                             device=dev)
            w_bytes = n * k
            self.copies = self._rotate(packed, w_bytes)
            self.dtype = "fp8"
            out = torch.empty((mmax, n), dtype=torch.bfloat16, device=dev)
            # fp32 A read by the quantizer (twice: amax, cast), codes written and
            # read, B, C
            alg = w_bytes + 8 * mmax * k + 2 * mmax * k + 2 * mmax * n
            self.calls.append((lambda c: qg.qgemm_fp8_act(a_d, self.copies[c], sb, n, workspace=ws,
                                                          out=out),
                               alg, w_bytes, 2 * mmax * n * k))
        elif fmt == "mxfp4_act":
            a, w = wl.mxfp4_operands(mmax, n, k)
            wc, we = qg.qgemm_quantize_mxfp4(torch.from_numpy(w).to(dev))
            del w
            packed = qg.qgemm_prepack("mxfp4", wc, k, n, w_scales=we)
            del wc, we
            a_d = torch.from_numpy(a).to(dev)
            del a
            ws = torch.empty(qg.qgemm_act_workspace_bytes("mxfp4", mmax, k), dtype=torch.uint8,
                             device=dev)
            w_bytes = n * k // 2 + n * k // 32
            a_bytes = 4 * mmax * k
            self.copies = self._rotate(packed, w_bytes + a_bytes)
            self.a_copies = [a_d] + [a_d.clone() for _ in range(len(self.copies) - 1)]
            self.dtype = "fp4"
            out = torch.empty((mmax, n), dtype=torch.bfloat16, device=dev)
            alg = w_bytes + a_bytes + (mmax * k // 2 + mmax * k // 32) * 2 + 2 * mmax * n
            self.calls.append((lambda c: qg.qgemm_mxfp4_act(self.a_copies[c], self.copies[c], n,
                                                            workspace=ws, out=out),
                               alg, w_bytes, 2 * mmax * n * k))
        elif fmt == "mxfp4":
            a, w = wl.mxfp4_operands(mmax, n, k)
            ac, ae = qg.qgemm_quantize_mxfp4(torch.from_numpy(a).to(dev))
            wc, we = qg.qgemm_quantize_mxfp4(torch.from_numpy(w).to(dev))
            del a, w
            packed = qg.qgemm_prepack("mxfp4", wc, k, n, w_scales=we)
            del wc, we
            w_bytes = n * k // 2 + n * k // 32
            a_bytes = mmax * k // 2 + mmax * k // 32
            self.copies = self._rotate(packed, w_bytes + a_bytes)
            self.a_copies = [ac] + [ac.clone() for _ in range(len(self.copies) - 1)]
            self.dtype = "fp4"
            for m in ms:
                out = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
                aem = ae[:m]
                alg = w_bytes + m * k // 2 + m * k // 32 + 2 * m * n
                self.calls.append((lambda c, m=m, aem=aem, out=out: qg.qgemm_mxfp4(
                    self.a_copies[c][:m], aem, self.copies[c], n, out=out),
                    alg, w_bytes, 2 * m * n * k))
        elif fmt == "fp8":
            a, b = wl.fp8_operands(mmax, n, k)
            qa, sa = qg.qgemm_quantize_fp8(torch.from_numpy(a).to(dev))
            qb, sb = qg.qgemm_quantize_fp8(torch.from_numpy(b).to(dev))
            del a, b
            packed = qg.qgemm_prepack("fp8", qb, k, n)
            del qb
            w_bytes = n * k
            a_bytes = mmax * k
            self.copies = self._rotate(packed, w_bytes + a_bytes)
            self.a_copies = [qa] + [qa.clone() for _ in range(len(self.copies) - 1)]
            self.dtype = "fp8"
            for m in ms:
                out = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
                alg = w_bytes + m * k + 2 * m * n
                self.calls.append((lambda c, m=m, out=out: qg.qgemm_fp8(
                    self.a_copies[c][:m], self.copies[c], sa, sb, n, out=out),
                    alg, w_bytes, 2 * m * n * k))
        torch.cuda.synchronize()

    @staticmethod
    def _rotate(packed, bytes_per_copy):
        r = max(1, math.ceil(ROTATE_BYTES / max(bytes_per_copy, 1)))
        return [packed] + [packed.clone() for _ in range(r - 1)]

    def enqueue_step(self, step):
        """Enqueue one step; call j of step i uses weight copy (len(calls)*i + j) % R."""
        per = len(self.calls)
        r = len(self.copies)
        for j, (launch, _, _, _) in enumerate(self.calls):
            launch((per * step + j) % r)

    def per_step(self):
        alg = sum(c[1] for c in self.calls)
        wgt = sum(c[2] for c in self.calls)
        flops = sum(c[3] for c in self.calls)
        return alg, wgt, flops


# ---------------------------------------------------------------------------
# timing
# ---------------------------------------------------------------------------

def time_steps(setup, steps, warmup, use_graph=True):
    import torch

    for i in range(warmup):
        setup.enqueue_step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    graph = None
    if use_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(steps):
                setup.enqueue_step(i)
        torch.cuda.synchronize()
        graph.replay()              # one untimed replay: first-launch costs
        torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    if graph is not None:
        graph.replay()
    else:
        for i in range(steps):
            setup.enqueue_step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return t1 - t0, ev0.elapsed_time(ev1) / 1e3


def per_call_times(setup, reps=60, warm=False):
    """Average device time of each call on its own (graph of `reps` calls).

    Cold (default): the calls rotate over the operand copies, so HBM serves
    them.  warm: every call reads copy 0, which then stays in the caches (the
    decode weights and the square GEMMs' operands fit the 256 MB Infinity
    Cache)."""
    import torch

    out = []
    r = 1 if warm else len(setup.copies)
    for launch, alg, wgt, flops in setup.calls:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(reps):
                launch(i % r)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) / 1e3 / reps)
    return out


def time_callable(fn, reps=20):
    """Average device time of a torch callable (HIP events on the current stream)."""
    import torch

    fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / 1e3 / reps


def read_ceiling(nbytes, reps=60, grids=(256, 512, 1024, 2048)):
    """The plain streaming-read reference for `nbytes` of weight: the library's
    read probe over rotating copies totalling >= ROTATE_BYTES (cold cache, as
    the GEMMs see their weights), timed like the GEMM calls (a graph of
    `reps` launches between HIP events on the launch stream); the fastest of a
    few grid sizes."""
    import torch
    import bit_quantized_gemm_qgemm_amd as qg

    n = -(-int(nbytes) // 16) * 16
    r = max(2, math.ceil(ROTATE_BYTES / n))
    bufs = [torch.randint(0, 255, (n,), dtype=torch.uint8, device="cuda") for _ in range(r)]
    sink = torch.empty(max(grids), dtype=torch.int32, device="cuda")
    best = None
    for wgs in grids:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(reps):
                qg.qgemm_read_probe(bufs[i % r], sink, wgs)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / 1e3 / reps
        if best is None or t < best[0]:
            best = (t, wgs)
    del bufs, sink
    torch.cuda.empty_cache()
    t, wgs = best
    return {"bytes": n, "us": round(t * 1e6, 3), "GBps": round(n / t / 1e9, 1),
            "frac_of_peak": round(n / t / 1e9 / HBM_PEAK_GBS, 4), "workgroups": wgs,
            "kernel": "read_probe_kernel (qgemm_read_probe)"}


def mfma_ceiling(dtype, launches=10, workgroups=256):
    """The practical rate of the scaled 32x32x64 matrix instruction on this GPU:
    the library's matrix-pipe probe (register operands of random bytes, no
    other instruction in its loop) over a graph of `launches` launches of about
    a millisecond each, timed like the GEMM calls."""
    import torch
    import bit_quantized_gemm_qgemm_amd as qg

    fp4 = dtype == "fp4"
    iters = 4096 if fp4 else 2048
    g = torch.Generator(device="cuda").manual_seed(0)
    ops = torch.randint(0, 256, (272 * 256 * workgroups,), generator=g, dtype=torch.uint8,
                        device="cuda")
    if not fp4:
        ops[(ops & 0x7F) == 0x7F] -= 1           # no e4m3 NaN codes
    sink = torch.empty(workgroups, dtype=torch.float32, device="cuda")
    fmt = "mxfp4" if fp4 else "fp8"
    qg.qgemm_mfma_probe(fmt, ops, iters, sink, workgroups)
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        for _ in range(launches):
            qg.qgemm_mfma_probe(fmt, ops, iters, sink, workgroups)
    gr.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    gr.replay()
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / 1e3 / launches
    flops = workgroups * 4 * iters * 16 * 131072
    tf = flops / t / 1e12
    return {"TFLOPS": round(tf, 1), "frac_of_peak": round(tf / MFMA_PEAK_TFLOPS[dtype], 4),
            "us_per_launch": round(t * 1e6, 1), "iters": iters, "workgroups": workgroups,
            "kernel": "mfma_probe_kernel (qgemm_mfma_probe)"}


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on the host
# ---------------------------------------------------------------------------

def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return 1


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(name, budget_s=10.0):
    import oracle
    import qgemm_workloads as wl

    fmt, ms, n, k = WORKLOADS[name]
    mmax = max(ms)
    if fmt in ("w4a16_grouped", "w8a16_grouped") and mmax <= SMALL_M_MAX:
        w4 = fmt == "w4a16_grouped"
        gen = wl.w4a16_grouped if w4 else wl.w8a16_grouped
        ggemm = oracle.gemm_w4a16_grouped if w4 else oracle.gemm_w8a16_grouped
        cols = n if k * n <= 50_000_000 else max(16, int(50_000_000 // k))
        x, w, s, z = gen(mmax, k, n, GROUP_K)
        w, s, z = np.ascontiguousarray(w[:, :cols]), s[:, :cols], z[:, :cols]
        gemm = lambda xm, w, s: ggemm(xm, w, s, z, GROUP_K)  # noqa: E731
        w_bytes_per_step = sum(((k * cols // 2) if w4 else k * cols) + 3 * s.size for _ in ms)
    if fmt == "nvfp4" and mmax <= SMALL_M_MAX:
        cols = n if k * n <= 50_000_000 else max(16, int(50_000_000 // k))
        x, codes, scales, g = wl.nvfp4_weight(mmax, k, n)
        w, s = np.ascontiguousarray(codes[:cols]), np.ascontiguousarray(scales[:cols])
        gemm = lambda xm, w, s: oracle.gemm_nvfp4(xm, w, s, g)  # noqa: E731
        w_bytes_per_step = sum(k * cols // 2 + k * cols // 16 for _ in ms)
    if fmt in ("mxfp4", "fp8") and mmax <= SMALL_M_MAX:
        # bounded sample: the full K and a column slice sized for ~1 s per step
        cols = max(16, int(20_000_000 // k))
        if fmt == "mxfp4":
            a, wt = wl.mxfp4_operands(mmax, cols, k)
            ac, ae = oracle.mxfp4_quantize(a)
            wc, we = oracle.mxfp4_quantize(wt)
            gemm = lambda xm, w, s: oracle.gemm_mxfp4(ac[:len(xm)], ae[:len(xm)], wc, we)  # noqa: E731
            w_bytes_per_step = sum(k * cols // 2 + k * cols // 32 for _ in ms)
        else:
            a, b = wl.fp8_operands(mmax, cols, k)
            qa, sa = oracle.fp8_quantize(a)
            qb, sb = oracle.fp8_quantize(b)
            gemm = lambda xm, w, s: oracle.gemm_fp8(qa[:len(xm)], qb, sa, sb)  # noqa: E731
            w_bytes_per_step = sum(k * cols for _ in ms)
        x, w, s = a, None, None
    if fmt in ("w4a16", "w8a16", "w4a16_grouped", "w8a16_grouped", "nvfp4", "mxfp4", "fp8") \
            and mmax <= SMALL_M_MAX:
        if fmt in ("w4a16", "w8a16"):
            gen = wl.w4a16 if fmt == "w4a16" else wl.w8a16
            gemm = oracle.gemm_w4a16 if fmt == "w4a16" else oracle.gemm_w8a16
            # bounded sample: the full K and a column slice sized for ~1 s per step
            cols = n if k * n <= 50_000_000 else max(16, int(50_000_000 // k))
            x, w, s = gen(mmax, k, n)
            w, s = np.ascontiguousarray(w[:, :cols]), s[:cols]
            w_bytes_per_step = sum(((k * cols // 2) if fmt == "w4a16" else k * cols) + 2 * cols
                                   for _ in ms)
        unit, done, t0 = "GB/s", 0, time.perf_counter()
        while True:
            for m in ms:
                gemm(x[:m], w, s)
            done += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        dt = time.perf_counter() - t0
        value = w_bytes_per_step * done / dt / 1e9
        sample = (f"oracle {fmt} steps (M={list(ms)}), K={k}, {cols} of {n} columns, "
                  f"{done} steps in {dt:.1f} s")
    elif fmt == "fp8_act":
        # quantize the whole A with the oracle, then the GEMM against a column slice
        cols = 512
        a, b = wl.fp8_operands(mmax, n, k)
        qb, sb = oracle.fp8_quantize(b[:, :cols])
        unit, done, t0 = "GB/s", 0, time.perf_counter()
        while True:
            qa, sa = oracle.fp8_quantize(a)
            oracle.gemm_fp8(qa, qb, sa, sb)
            done += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        dt = time.perf_counter() - t0
        value = k * cols * done / dt / 1e9
        sample = (f"oracle fp8 quantize of A [{mmax}, {k}] + GEMM against {cols} of {n} columns, "
                  f"{done} runs in {dt:.1f} s")
    else:
        # bounded sample: 256 rows of X / A against the whole weight
        rows = 256
        unit = "TFLOP/s"
        if fmt in ("w4a16", "w8a16"):
            gen = wl.w4a16 if fmt == "w4a16" else wl.w8a16
            gemm = oracle.gemm_w4a16 if fmt == "w4a16" else oracle.gemm_w8a16
            x, w, s = gen(rows, k, n)
            run = lambda: gemm(x, w, s)  # noqa: E731
        elif fmt in ("w4a16_grouped", "w8a16_grouped"):
            w4 = fmt == "w4a16_grouped"
            gen = wl.w4a16_grouped if w4 else wl.w8a16_grouped
            ggemm = oracle.gemm_w4a16_grouped if w4 else oracle.gemm_w8a16_grouped
            x, w, s, z = gen(rows, k, n, GROUP_K)
            run = lambda: ggemm(x, w, s, z, GROUP_K)  # noqa: E731
        elif fmt == "nvfp4":
            x, codes, scales, g = wl.nvfp4_weight(rows, k, n)
            run = lambda: oracle.gemm_nvfp4(x, codes, scales, g)  # noqa: E731
        elif fmt in ("mxfp4", "mxfp4_act"):
            a, w = wl.mxfp4_operands(rows, n, k)
            ac, ae = oracle.mxfp4_quantize(a)
            wc, we = oracle.mxfp4_quantize(w)
            if fmt == "mxfp4_act":   # the activation quantizer is part of each run
                def run():
                    c_, e_ = oracle.mxfp4_quantize(a)
                    return oracle.gemm_mxfp4(c_, e_, wc, we)
            else:
                run = lambda: oracle.gemm_mxfp4(ac, ae, wc, we)  # noqa: E731
        else:
            a, b = wl.fp8_operands(rows, n, k)
            qa, sa = oracle.fp8_quantize(a)
            qb, sb = oracle.fp8_quantize(b)
            run = lambda: oracle.gemm_fp8(qa, qb, sa, sb)  # noqa: E731
        done, t0 = 0, time.perf_counter()
        while True:
            run()
            done += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        dt = time.perf_counter() - t0
        value = 2.0 * rows * n * k * done / dt / 1e12
        sample = (f"oracle {fmt} GEMM of {rows} x {k} by {k} x {n} (dequantize + fp64 matmul), "
                  f"{done} runs in {dt:.1f} s")
    # cores = the BLAS threads the oracle's matmul ran on; the host's model and
    # the CPUs this process may use are stated beside it
    return {"value": value, "unit": unit, "cores": blas_threads(), "kind": "oracle",
            "sample": sample, "cpu_model": cpu_model(),
            "affinity_cpus": len(os.sched_getaffinity(0))}


# ---------------------------------------------------------------------------

def traffic_for(kernel):
    """HBM bytes per launch from committed rocprofv3 counter runs, or None when
    missing or taken on a different version of the kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
        ent = data.get(kernel)
        if ent and ent.get("source_sha") == source_hash(kernel):
            return ent["bytes_per_launch"]
    except (OSError, ValueError, KeyError, StopIteration):
        pass
    return None


def run(name, steps, warmup, with_cpu, use_graph, with_ceiling=True):
    import torch

    setup = Setup(name)
    alg, wgt, flops = setup.per_step()
    wall, dev_s = time_steps(setup, steps, warmup, use_graph=use_graph)
    per_call = per_call_times(setup)
    per_call_warm = per_call_times(setup, warm=True)
    decode = setup.kind == "decode"
    # the dominant kernel is the call with the longest average duration (of
    # calls within 2% of the longest, the one with the largest M, so that
    # near-ties do not flip between runs); each call's launches were timed
    # with HIP events on the launch stream
    longest = max(per_call)
    dom = max(i for i in range(len(setup.calls)) if per_call[i] >= 0.98 * longest)
    _, dom_alg, _, dom_flops = setup.calls[dom]
    if decode:
        value = wgt * steps / wall / 1e9
        unit = "GB/s"
        achieved = dom_alg / per_call[dom] / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS}
    else:
        value = flops * steps / wall / 1e12
        unit = "TFLOPS"
        achieved = dom_flops / per_call[dom] / 1e12
        peak = MFMA_PEAK_TFLOPS[setup.dtype]
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                "frac": achieved / peak}
    kernel = kernel_name(setup, setup.ms[dom])
    roof["traffic"] = traffic_for(kernel)
    roof["kernel"] = kernel
    roof["avg_launch_us"] = round(per_call[dom] * 1e6, 3)
    roof["step_avg_launch_us"] = round(dev_s / (steps * len(setup.calls)) * 1e6, 3)
    detail = []
    for (launch, a_b, w_b, fl), t, tw, m in zip(setup.calls, per_call, per_call_warm, setup.ms):
        d = {"M": m, "us": round(t * 1e6, 3), "weight_GBps": round(w_b / t / 1e9, 1),
             "alg_GBps": round(a_b / t / 1e9, 1), "TFLOPS": round(fl / t / 1e12, 2),
             "warm_us": round(tw * 1e6, 3)}
        d["pct_hbm"] = round(100 * a_b / t / 1e9 / HBM_PEAK_GBS, 1)
        if not decode:
            d["pct_mfma"] = round(100 * fl / t / 1e12 / MFMA_PEAK_TFLOPS[setup.dtype], 1)
        detail.append(d)
    if setup.explicit is not None:
        detail[0]["explicit_dequant_us"] = round(time_callable(setup.explicit) * 1e6, 3)
    ceiling = None
    if decode and with_ceiling:
        # the same weight byte count read by a plain streaming-read kernel
        ceiling = read_ceiling(setup.calls[dom][2])
        roof["frac_of_read_ceiling"] = round(ceiling["us"] / (per_call[dom] * 1e6), 4)
    mceiling = None
    if not decode and with_ceiling and setup.dtype in ("fp4", "fp8"):
        # the matrix instruction's own practical rate on this GPU
        mceiling = mfma_ceiling(setup.dtype)
        roof["frac_of_mfma_ceiling"] = round(achieved / mceiling["TFLOPS"], 4)
    cfg = {"workload": name, "format": setup.fmt, "M": list(setup.ms), "N": setup.n,
           "K": setup.k, "weight_copies": len(setup.copies),
           "timing": "hip-graph replay" if use_graph else "eager launches"}
    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": unit,
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(wall / steps * 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": setup.dtype,
        "data": "synthetic (seeded NumPy draws in the workloads' shapes and distributions)",
        "config": cfg,
        "roofline": roof,
        "detail": detail,
        "device": torch.cuda.get_device_name(0),
    }
    if ceiling is not None:
        line["read_ceiling"] = ceiling
    if mceiling is not None:
        line["mfma_ceiling"] = mceiling
    if with_cpu:
        line["cpu_baseline"] = cpu_baseline(name)
    del setup
    torch.cuda.empty_cache()
    return line


# The configurations the metric is quoted on besides the default one: the
# small W4A16 case, W4A16 decode, the 8192^3 MXFP4 and FP8 GEMMs and FP8 at
# decode M.  The default run times each the same way (graph replay of the
# timed steps, per-call HIP events) and reports them under "configs".
OTHER_CONFIGS = ("w4a16_small", "w4a16_decode", "mxfp4_square", "fp8_square", "fp8_decode")


def config_summary(line):
    """The parts of a workload's line that the default line carries per config."""
    r = line["roofline"]
    out = {"workload": line["config"]["workload"], "value": line["value"], "unit": line["unit"],
           "ms_per_step": line["ms_per_step"], "steps": line["steps"], "dtype": line["dtype"],
           "kernel": r["kernel"], "avg_launch_us": r["avg_launch_us"],
           "roofline_bound": r["bound"], "roofline_frac": round(r["frac"], 4),
           "per_call": line["detail"]}
    if "read_ceiling" in line:
        out["read_ceiling"] = line["read_ceiling"]
        out["frac_of_read_ceiling"] = r["frac_of_read_ceiling"]
    if "mfma_ceiling" in line:
        out["mfma_ceiling"] = line["mfma_ceiling"]
        out["frac_of_mfma_ceiling"] = r["frac_of_mfma_ceiling"]
    return out


def kernel_name(setup, m):
    """Label of the kernel that runs a call with M rows, as the library's own
    dispatch query names it (rocprofv3 lists the mangled template instance)."""
    import bit_quantized_gemm_qgemm_amd as qg
    fmt = {"fp8_act": "fp8", "mxfp4_act": "mxfp4"}.get(setup.fmt, setup.fmt)
    group_k = GROUP_K if fmt in ("w4a16_grouped", "w8a16_grouped") else 0
    name = qg.qgemm_dispatch_kernel(fmt, m, setup.n, setup.k, group_k)
    label = f"{name}[{fmt}, M={m}, N={setup.n}, K={setup.k}]"
    if setup.fmt == "fp8_act":
        return "qgemm_fp8_act call: quantize kernels + " + label
    if setup.fmt == "mxfp4_act":
        return "qgemm_mxfp4_act call: quantize_mxfp4_kernel + " + label
    return label


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(WORKLOADS))
    ap.add_argument("--all", action="store_true", help="one JSON line per workload")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--eager", action="store_true", help="launch eagerly instead of a graph")
    ap.add_argument("--no-configs", action="store_true",
                    help="default workload only: skip the other configurations' summaries")
    ap.add_argument("--calib-copy", action="store_true",
                    help="first run 4 plain device copies of 256 MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path; its "
              "kernels run one GPU's share of a column-parallel (decode) or output-tile "
              "(square GEMM) split, which needs no exchange between GPUs.",
              file=sys.stderr)
        sys.exit(2)
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.calib_copy:
        src = torch.empty(CALIB_BYTES, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"bench: ran 4 copies of {CALIB_BYTES} bytes for counter calibration")
    def steps_for(name):
        square = WORKLOADS[name][1][0] > 16
        steps = args.steps if args.steps is not None else (20 if square else 200)
        warmup = args.warmup if args.warmup is not None else (3 if square else 20)
        return steps, warmup

    names = sorted(WORKLOADS) if args.all else [args.workload]
    for name in names:
        steps, warmup = steps_for(name)
        log(f"bench: {name} steps={steps} warmup={warmup}")
        line = run(name, steps, warmup, with_cpu=not args.no_cpu, use_graph=not args.eager)
        if name == DEFAULT_WORKLOAD and not args.all and not args.no_configs:
            configs = []
            for other in OTHER_CONFIGS:
                o_steps, o_warmup = steps_for(other)
                # at least as many steps as the default line, at most 20 for the
                # square GEMMs (each step is a 0.3-0.5 ms call)
                o_steps = min(o_steps, 20) if WORKLOADS[other][1][0] > 16 else o_steps
                log(f"bench: {other} steps={o_steps} warmup={o_warmup} (config summary)")
                o = run(other, o_steps, o_warmup, with_cpu=False, use_graph=not args.eager)
                configs.append(config_summary(o))
            line["configs"] = configs
        print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
