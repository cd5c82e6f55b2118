"""Python binding of libqgemm (quantized GEMMs dequantized inside the kernel).

Argument marshalling only: each function checks dtypes and shapes of torch
tensors, allocates outputs with torch, and calls the C entry point of the same
name on torch's current stream.  Every step of the computation runs in the
library's HIP kernels; there is no fallback.  If libqgemm.so is missing the
calls raise instead of computing anything.
"""

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqgemm.so")

QGEMM_W4A16 = 1
QGEMM_W8A16 = 2
QGEMM_MXFP4 = 3
QGEMM_FP8 = 4
QGEMM_W4A16_GROUPED = 5
QGEMM_W8A16_GROUPED = 6
QGEMM_NVFP4 = 7

FORMATS = {"w4a16": QGEMM_W4A16, "w8a16": QGEMM_W8A16, "mxfp4": QGEMM_MXFP4, "fp8": QGEMM_FP8,
           "w4a16_grouped": QGEMM_W4A16_GROUPED, "w8a16_grouped": QGEMM_W8A16_GROUPED,
           "nvfp4": QGEMM_NVFP4}

# (name, restype, argtypes) of every symbol declared in include/qgemm.h
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_SIGNATURES = [
    ("qgemm_status_string", ctypes.c_char_p, [ctypes.c_int]),
    ("qgemm_abi_version", ctypes.c_int, []),
    ("qgemm_dispatch_kernel", ctypes.c_int, [ctypes.c_int, _I64, _I64, _I64, _I64]),
    ("qgemm_prepack_bytes", ctypes.c_int64, [ctypes.c_int, _I64, _I64]),
    ("qgemm_prepack", ctypes.c_int, [ctypes.c_int, _P, _P, _P, _I64, _I64, _P]),
    ("qgemm_quantize_mxfp4", ctypes.c_int, [_P, _I64, _I64, _P, _P, _P]),
    ("qgemm_quantize_fp8", ctypes.c_int, [_P, _I64, _P, _P, _P]),
    ("qgemm_w4a16", ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, _I64, _P]),
    ("qgemm_w8a16", ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, _I64, _P]),
    ("qgemm_mxfp4", ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, _I64, _P]),
    ("qgemm_fp8", ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _P]),
    ("qgemm_prepack_grouped_bytes", ctypes.c_int64, [ctypes.c_int, _I64, _I64, _I64]),
    ("qgemm_prepack_grouped", ctypes.c_int,
     [ctypes.c_int, _P, _P, _P, _I64, _I64, _P, _I64, _I64, _P]),
    ("qgemm_w4a16_grouped", ctypes.c_int, [_P, _P, _P, _I64, _I64, _I64, _I64, _P]),
    ("qgemm_w8a16_grouped", ctypes.c_int, [_P, _P, _P, _I64, _I64, _I64, _I64, _P]),
    ("qgemm_nvfp4", ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, _I64, _P]),
    ("qgemm_act_workspace_bytes", ctypes.c_int64, [ctypes.c_int, _I64, _I64]),
    ("qgemm_mxfp4_act", ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, _I64, _P]),
    ("qgemm_fp8_act", ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _P]),
    ("qgemm_fp8_act_noalloc", ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, _I64, _P]),
    ("qgemm_read_probe", ctypes.c_int, [_P, _I64, _P, _I64, _P]),
    ("qgemm_mfma_probe", ctypes.c_int, [ctypes.c_int, _P, _I64, _P, _I64, _P]),
]

# largest M * K that qgemm_fp8_act_noalloc accepts (its fixed scratch)
FP8_ACT_NOALLOC_MAX_ELEMS = 16 * 1024 * 1024

_lib = None


class QgemmError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: status {status} ({status_string(status)})")


def lib():
    """The loaded libqgemm.so (ctypes), loading it on first use."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m bit_quantized_gemm_qgemm_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, res, args in _SIGNATURES:
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_string(status):
    return lib().qgemm_status_string(int(status)).decode()


def _check(status, where):
    if status != 0:
        raise QgemmError(status, where)


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _need(t, dtype, ndim, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got {t.dim()}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (row-major, no padding)")


def _out(out, M, N, dtype, device):
    """The caller's output tensor, checked to be a contiguous [M, N] device
    tensor of `dtype` (the library writes M * N elements through its pointer),
    or a new one."""
    if out is None:
        return torch.empty((M, N), dtype=dtype, device=device)
    _need(out, dtype, 2, "out")
    if tuple(out.shape) != (M, N):
        raise ValueError(f"out must be [{M}, {N}], got {list(out.shape)}")
    return out


# qgemm_dispatch_kernel results: the kernel each launches, by its name in
# profiler traces
KERNELS = {0: None, 1: "decode_gemm_kernel", 2: "pipe256_kernel", 3: "mxw_kernel",
           4: "f8w_kernel", 5: "tile_gemm_kernel"}


def qgemm_dispatch_kernel(fmt, M, N, K, group_k=0):
    """Name of the kernel a GEMM call of this format and sizes launches (None
    when M or N is 0); host-only.  The fused-quantization calls dispatch as
    "mxfp4" / "fp8"."""
    st = lib().qgemm_dispatch_kernel(int(FORMATS.get(fmt, fmt)), int(M), int(N), int(K),
                                     int(group_k))
    if st < 0:
        raise QgemmError(int(st), "qgemm_dispatch_kernel")
    return KERNELS[st]


def qgemm_prepack_bytes(fmt, K, N):
    n = lib().qgemm_prepack_bytes(int(fmt), int(K), int(N))
    if n < 0:
        raise QgemmError(int(n), "qgemm_prepack_bytes")
    return int(n)


def qgemm_prepack(fmt, w, K, N, w_scales=None):
    """Canonical weight (device tensor) -> opaque packed uint8 device tensor."""
    fmt = FORMATS.get(fmt, fmt)
    if fmt == QGEMM_W4A16:
        _need(w, torch.uint8, 2, "w")
        if tuple(w.shape) != (K // 2, N) or K % 2:
            raise ValueError("W4A16 weight must be uint8 [K/2, N] with K even")
    elif fmt == QGEMM_W8A16:
        _need(w, torch.int8, 2, "w")
        if tuple(w.shape) != (K, N):
            raise ValueError("W8A16 weight must be int8 [K, N]")
    elif fmt == QGEMM_MXFP4:
        _need(w, torch.uint8, 2, "w")
        _need(w_scales, torch.uint8, 2, "w_scales")
        if tuple(w.shape) != (N, K // 2) or tuple(w_scales.shape) != (N, K // 32):
            raise ValueError("MXFP4 weight must be codes uint8 [N, K/2] and scales uint8 [N, K/32]")
    elif fmt == QGEMM_NVFP4:
        _need(w, torch.uint8, 2, "w")
        _need(w_scales, torch.uint8, 2, "w_scales")
        if tuple(w.shape) != (N, K // 2) or tuple(w_scales.shape) != (N, K // 16) or K % 16:
            raise ValueError("NVFP4 weight must be codes uint8 [N, K/2] and e4m3 scales "
                             "uint8 [N, K/16], K a multiple of 16")
    elif fmt == QGEMM_FP8:
        if w.dtype == torch.float8_e4m3fn:
            w = w.view(torch.uint8)
        _need(w, torch.uint8, 2, "w")
        if tuple(w.shape) != (K, N):
            raise ValueError("FP8 weight must be e4m3fn [K, N]")
    else:
        raise ValueError(f"unknown format {fmt}")
    nbytes = qgemm_prepack_bytes(fmt, K, N)
    out = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=w.device)
    _check(lib().qgemm_prepack(fmt, _ptr(w), _ptr(w_scales), _ptr(out), int(K), int(N),
                               _stream(w)), "qgemm_prepack")
    return out


def qgemm_quantize_mxfp4(x):
    """fp32 [rows, K] -> (codes uint8 [rows, K/2], e8m0 uint8 [rows, K/32])."""
    _need(x, torch.float32, 2, "x")
    rows, k = x.shape
    if k % 32:
        raise ValueError("K must be a multiple of 32")
    codes = torch.empty((rows, k // 2), dtype=torch.uint8, device=x.device)
    e8m0 = torch.empty((rows, k // 32), dtype=torch.uint8, device=x.device)
    _check(lib().qgemm_quantize_mxfp4(_ptr(x), rows, k, _ptr(codes), _ptr(e8m0), _stream(x)),
           "qgemm_quantize_mxfp4")
    return codes, e8m0


def qgemm_quantize_fp8(x):
    """fp32 tensor -> (e4m3fn codes as uint8 of the same shape, fp32 scale [1])."""
    if not isinstance(x, torch.Tensor) or x.dtype != torch.float32 or not x.is_cuda \
            or not x.is_contiguous():
        raise TypeError("x must be a contiguous float32 device tensor")
    codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    scale = torch.empty(1, dtype=torch.float32, device=x.device)
    _check(lib().qgemm_quantize_fp8(_ptr(x), x.numel(), _ptr(codes), _ptr(scale), _stream(x)),
           "qgemm_quantize_fp8")
    return codes, scale


def _weight_only(name, x, w_packed, scales, N, out):
    _need(x, torch.float16, 2, "x")
    _need(w_packed, torch.uint8, 1, "w_packed")
    _need(scales, torch.float16, 1, "scales")
    M, K = x.shape
    if scales.shape[0] != N:
        raise ValueError("scales must have N entries")
    fmt = QGEMM_W4A16 if name == "qgemm_w4a16" else QGEMM_W8A16
    if w_packed.numel() < qgemm_prepack_bytes(fmt, K, N):
        raise ValueError("w_packed is smaller than the packed size for this K, N")
    out = _out(out, M, N, torch.float16, x.device)
    fn = getattr(lib(), name)
    _check(fn(_ptr(x), _ptr(w_packed), _ptr(scales), _ptr(out), M, N, K, _stream(x)), name)
    return out


def qgemm_w4a16(x, w_packed, scales, N, out=None):
    """Y = X @ ((code - 8) * s) -> fp16 [M, N]."""
    return _weight_only("qgemm_w4a16", x, w_packed, scales, N, out)


def qgemm_w8a16(x, w_packed, scales, N, out=None):
    """Y = X @ (w * s) -> fp16 [M, N]."""
    return _weight_only("qgemm_w8a16", x, w_packed, scales, N, out)


def qgemm_mxfp4(a_codes, a_e8m0, w_packed, N, out=None):
    """C = A_deq @ W_deq^T -> bf16 [M, N]."""
    _need(a_codes, torch.uint8, 2, "a_codes")
    _need(a_e8m0, torch.uint8, 2, "a_e8m0")
    _need(w_packed, torch.uint8, 1, "w_packed")
    M, half_k = a_codes.shape
    K = 2 * half_k
    if tuple(a_e8m0.shape) != (M, K // 32):
        raise ValueError("a_e8m0 must be [M, K/32]")
    if w_packed.numel() < qgemm_prepack_bytes(QGEMM_MXFP4, K, N):
        raise ValueError("w_packed is smaller than the packed size for this K, N")
    out = _out(out, M, N, torch.bfloat16, a_codes.device)
    _check(lib().qgemm_mxfp4(_ptr(a_codes), _ptr(a_e8m0), _ptr(w_packed), _ptr(out), M, N, K,
                             _stream(a_codes)), "qgemm_mxfp4")
    return out


def qgemm_fp8(a, b_packed, scale_a, scale_b, N, out=None):
    """C = (A @ B) * scale_a * scale_b -> bf16 [M, N]; scales are device fp32 [1]."""
    if a.dtype == torch.float8_e4m3fn:
        a = a.view(torch.uint8)
    _need(a, torch.uint8, 2, "a")
    _need(b_packed, torch.uint8, 1, "b_packed")
    for s, nm in ((scale_a, "scale_a"), (scale_b, "scale_b")):
        if s.dtype != torch.float32 or not s.is_cuda or s.numel() != 1:
            raise TypeError(f"{nm} must be a one-element float32 device tensor")
    M, K = a.shape
    if b_packed.numel() < qgemm_prepack_bytes(QGEMM_FP8, K, N):
        raise ValueError("b_packed is smaller than the packed size for this K, N")
    out = _out(out, M, N, torch.bfloat16, a.device)
    _check(lib().qgemm_fp8(_ptr(a), _ptr(b_packed), _ptr(scale_a), _ptr(scale_b), _ptr(out), M,
                           N, K, _stream(a)), "qgemm_fp8")
    return out


def qgemm_prepack_grouped_bytes(fmt, K, N, group_k):
    n = lib().qgemm_prepack_grouped_bytes(int(FORMATS.get(fmt, fmt)), int(K), int(N), int(group_k))
    if n < 0:
        raise QgemmError(int(n), "qgemm_prepack_grouped_bytes")
    return int(n)


def qgemm_prepack_grouped(fmt, w, K, N, scales, zeros=None, group_k=128, group_n=1):
    """Codes + group-wise fp16 scales [ceil(K/group_k), ceil(N/group_n)] (+ zero
    points of the same shape: uint8 0..15 for W4, int8 for W8; None for the
    symmetric 8 / 0) -> opaque packed uint8 device tensor."""
    fmt = FORMATS.get(fmt, fmt)
    if fmt == QGEMM_W4A16_GROUPED:
        _need(w, torch.uint8, 2, "w")
        if tuple(w.shape) != (K // 2, N):
            raise ValueError("grouped W4A16 weight must be uint8 [K/2, N]")
        zdtype = torch.uint8
    elif fmt == QGEMM_W8A16_GROUPED:
        _need(w, torch.int8, 2, "w")
        if tuple(w.shape) != (K, N):
            raise ValueError("grouped W8A16 weight must be int8 [K, N]")
        zdtype = torch.int8
    else:
        raise ValueError(f"not a grouped format: {fmt}")
    shape = (-(-K // group_k), -(-N // group_n))
    _need(scales, torch.float16, 2, "scales")
    if tuple(scales.shape) != shape:
        raise ValueError(f"scales must be {shape}")
    if zeros is not None:
        _need(zeros, zdtype, 2, "zeros")
        if tuple(zeros.shape) != shape:
            raise ValueError(f"zeros must be {shape}")
    nbytes = qgemm_prepack_grouped_bytes(fmt, K, N, group_k)
    out = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=w.device)
    _check(lib().qgemm_prepack_grouped(fmt, _ptr(w), _ptr(scales), _ptr(zeros), int(group_k),
                                       int(group_n), _ptr(out), int(K), int(N), _stream(w)),
           "qgemm_prepack_grouped")
    return out


def _grouped(name, fmt, x, w_packed, N, group_k, out):
    _need(x, torch.float16, 2, "x")
    _need(w_packed, torch.uint8, 1, "w_packed")
    M, K = x.shape
    if w_packed.numel() < qgemm_prepack_grouped_bytes(fmt, K, N, group_k):
        raise ValueError("w_packed is smaller than the packed size for this K, N, group_k")
    out = _out(out, M, N, torch.float16, x.device)
    _check(getattr(lib(), name)(_ptr(x), _ptr(w_packed), _ptr(out), M, N, K, int(group_k),
                                _stream(x)), name)
    return out


def qgemm_w4a16_grouped(x, w_packed, N, group_k, out=None):
    """Y = X @ ((code - z) * s) with group-wise s, z -> fp16 [M, N]."""
    return _grouped("qgemm_w4a16_grouped", QGEMM_W4A16_GROUPED, x, w_packed, N, group_k, out)


def qgemm_w8a16_grouped(x, w_packed, N, group_k, out=None):
    """Y = X @ ((w - z) * s) with group-wise s, z -> fp16 [M, N]."""
    return _grouped("qgemm_w8a16_grouped", QGEMM_W8A16_GROUPED, x, w_packed, N, group_k, out)


def qgemm_nvfp4(x, w_packed, global_scale, N, out=None):
    """Y = X @ (e2m1 * e4m3 block scale * global)^T -> fp16 [M, N]; global_scale
    is a one-element float32 device tensor."""
    _need(x, torch.float16, 2, "x")
    _need(w_packed, torch.uint8, 1, "w_packed")
    if global_scale.dtype != torch.float32 or not global_scale.is_cuda or global_scale.numel() != 1:
        raise TypeError("global_scale must be a one-element float32 device tensor")
    M, K = x.shape
    if w_packed.numel() < qgemm_prepack_bytes(QGEMM_NVFP4, K, N):
        raise ValueError("w_packed is smaller than the packed size for this K, N")
    out = _out(out, M, N, torch.float16, x.device)
    _check(lib().qgemm_nvfp4(_ptr(x), _ptr(w_packed), _ptr(global_scale), _ptr(out), M, N, K,
                             _stream(x)), "qgemm_nvfp4")
    return out


def qgemm_act_workspace_bytes(fmt, M, K):
    n = lib().qgemm_act_workspace_bytes(int(FORMATS.get(fmt, fmt)), int(M), int(K))
    if n < 0:
        raise QgemmError(int(n), "qgemm_act_workspace_bytes")
    return int(n)


def _act_workspace(fmt, a, workspace):
    M, K = a.shape
    need = qgemm_act_workspace_bytes(fmt, M, K)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=a.device)
    else:
        _need(workspace, torch.uint8, 1, "workspace")
        if workspace.numel() < need:
            raise ValueError(f"workspace needs {need} bytes")
    return workspace


def qgemm_mxfp4_act(a, w_packed, N, workspace=None, out=None):
    """fp32 A [M, K] -> MXFP4 on the device, then C = A_deq @ W_deq^T (bf16).
    Returns (C, workspace); the workspace holds the quantized A."""
    _need(a, torch.float32, 2, "a")
    _need(w_packed, torch.uint8, 1, "w_packed")
    M, K = a.shape
    if w_packed.numel() < qgemm_prepack_bytes(QGEMM_MXFP4, K, N):
        raise ValueError("w_packed is smaller than the packed size for this K, N")
    workspace = _act_workspace(QGEMM_MXFP4, a, workspace)
    out = _out(out, M, N, torch.bfloat16, a.device)
    _check(lib().qgemm_mxfp4_act(_ptr(a), _ptr(w_packed), _ptr(out), _ptr(workspace), M, N, K,
                                 _stream(a)), "qgemm_mxfp4_act")
    return out, workspace


def qgemm_fp8_act(a, b_packed, scale_b, N, workspace=None, out=None):
    """fp32 A [M, K] -> per-tensor e4m3fn on the device, then C = (A_q @ B) *
    s_a * s_b (bf16).  Returns (C, workspace); the workspace holds the codes
    and, at round_up(M*K, 16), the fp32 scale."""
    _need(a, torch.float32, 2, "a")
    _need(b_packed, torch.uint8, 1, "b_packed")
    if scale_b.dtype != torch.float32 or not scale_b.is_cuda or scale_b.numel() != 1:
        raise TypeError("scale_b must be a one-element float32 device tensor")
    M, K = a.shape
    if b_packed.numel() < qgemm_prepack_bytes(QGEMM_FP8, K, N):
        raise ValueError("b_packed is smaller than the packed size for this K, N")
    workspace = _act_workspace(QGEMM_FP8, a, workspace)
    out = _out(out, M, N, torch.bfloat16, a.device)
    _check(lib().qgemm_fp8_act(_ptr(a), _ptr(b_packed), _ptr(scale_b), _ptr(out), _ptr(workspace),
                               M, N, K, _stream(a)), "qgemm_fp8_act")
    return out, workspace


def qgemm_fp8_act_noalloc(a, b_packed, scale_b, N, out):
    """As qgemm_fp8_act, with the quantized A in the library's fixed per-GPU
    scratch instead of a workspace: the entry point allocates nothing, so the
    caller passes the output.  M * K <= FP8_ACT_NOALLOC_MAX_ELEMS."""
    _need(a, torch.float32, 2, "a")
    _need(b_packed, torch.uint8, 1, "b_packed")
    if scale_b.dtype != torch.float32 or not scale_b.is_cuda or scale_b.numel() != 1:
        raise TypeError("scale_b must be a one-element float32 device tensor")
    M, K = a.shape
    if b_packed.numel() < qgemm_prepack_bytes(QGEMM_FP8, K, N):
        raise ValueError("b_packed is smaller than the packed size for this K, N")
    if out is None:
        raise ValueError("qgemm_fp8_act_noalloc needs a caller-allocated out [M, N]")
    out = _out(out, M, N, torch.bfloat16, a.device)
    _check(lib().qgemm_fp8_act_noalloc(_ptr(a), _ptr(b_packed), _ptr(scale_b), _ptr(out), M, N,
                                       K, _stream(a)), "qgemm_fp8_act_noalloc")
    return out


def qgemm_read_probe(buf, sink, workgroups):
    """Read all of the uint8 device tensor `buf` once (the plain-read
    reference of the weight stream); sink is an int32 device tensor with at
    least `workgroups` entries."""
    _need(buf, torch.uint8, 1, "buf")
    _need(sink, torch.int32, 1, "sink")
    if sink.numel() < workgroups:
        raise ValueError("sink needs one entry per workgroup")
    _check(lib().qgemm_read_probe(_ptr(buf), buf.numel(), _ptr(sink), int(workgroups),
                                  _stream(buf)), "qgemm_read_probe")


def qgemm_mfma_probe(fmt, operands, iters, sink, workgroups):
    """Back-to-back scaled matrix instructions on register operands loaded from
    the uint8 device tensor `operands` (272 bytes per thread); sink is a
    float32 device tensor with at least `workgroups` entries."""
    _need(operands, torch.uint8, 1, "operands")
    _need(sink, torch.float32, 1, "sink")
    if operands.numel() < 272 * 256 * workgroups or sink.numel() < workgroups:
        raise ValueError("operands needs 272 bytes per thread, sink one entry per workgroup")
    _check(lib().qgemm_mfma_probe(int(FORMATS.get(fmt, fmt)), _ptr(operands), int(iters),
                                  _ptr(sink), int(workgroups), _stream(operands)),
           "qgemm_mfma_probe")
