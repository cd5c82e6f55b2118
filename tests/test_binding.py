"""Host-only tests of the Python binding's argument checks.

The binding checks dtypes and shapes before it calls into the library; a
caller-supplied output of the wrong shape would otherwise receive M * N
elements through its pointer.  These tests run without a GPU: host tensors
are made to pass the binding's device-tensor test, and the library handle is
a stand-in that answers the host-only size queries from the real library
and records (instead of running) every other call, so the tests see whether a
launch would have been attempted.
"""

import os

import pytest
import torch

import bit_quantized_gemm_qgemm_amd as qg


class RecordingLib:
    """Stand-in for the ctypes handle: size queries go to the real library,
    every other entry point records its name and returns OK."""

    HOST_ONLY = ("qgemm_prepack_bytes", "qgemm_prepack_grouped_bytes",
                 "qgemm_act_workspace_bytes", "qgemm_status_string")

    def __init__(self, real):
        self.real = real
        self.calls = []

    def __getattr__(self, name):
        if name in self.HOST_ONLY:
            return getattr(self.real, name)

        def record(*args):
            self.calls.append(name)
            return 0
        return record


@pytest.fixture
def fake(monkeypatch):
    if not os.path.exists(qg.LIB_PATH):
        from bit_quantized_gemm_qgemm_amd import build
        build.build()
    rec = RecordingLib(qg.lib())
    monkeypatch.setattr(qg, "lib", lambda: rec)
    monkeypatch.setattr(qg, "_stream", lambda t: None)
    # host tensors pass the binding's device-tensor checks unchanged
    monkeypatch.setattr(torch.Tensor, "is_cuda", property(lambda self: True), raising=False)
    return rec, torch.ones(1, dtype=torch.float32)


def u8(*shape):
    return torch.zeros(shape, dtype=torch.uint8)


def calls_for_shapes(fn, good, bad_shapes, dtype, rec):
    """fn(out) must run with `good` and raise ValueError, with no recorded
    call, for every wrong shape."""
    for shape in bad_shapes:
        before = len(rec.calls)
        with pytest.raises(ValueError, match=r"out must be"):
            fn(torch.zeros(shape, dtype=dtype))
        assert len(rec.calls) == before, f"launched with out {shape}"
    fn(torch.zeros(good, dtype=dtype))
    return rec.calls[-1]


M, N, K = 4, 32, 64
BAD = [(M, N - 1), (M - 1, N), (N, M), (1, M * N - 1)]


def test_mxfp4_out_shape_checked_before_launch(fake):
    rec, _ = fake
    wp = u8(qg.qgemm_prepack_bytes(3, K, N))
    name = calls_for_shapes(lambda out: qg.qgemm_mxfp4(u8(M, K // 2), u8(M, K // 32), wp, N,
                                                       out=out),
                            (M, N), BAD, torch.bfloat16, rec)
    assert name == "qgemm_mxfp4"


def test_fp8_out_shape_checked_before_launch(fake):
    rec, scalar = fake
    bp = u8(qg.qgemm_prepack_bytes(4, K, N))
    name = calls_for_shapes(lambda out: qg.qgemm_fp8(u8(M, K), bp, scalar, scalar, N, out=out),
                            (M, N), BAD, torch.bfloat16, rec)
    assert name == "qgemm_fp8"


def test_act_out_shape_checked_before_launch(fake):
    rec, scalar = fake
    a = torch.zeros((M, K), dtype=torch.float32)
    wp = u8(qg.qgemm_prepack_bytes(3, K, N))
    ws = u8(qg.qgemm_act_workspace_bytes("mxfp4", M, K))
    name = calls_for_shapes(lambda out: qg.qgemm_mxfp4_act(a, wp, N, workspace=ws, out=out),
                            (M, N), BAD, torch.bfloat16, rec)
    assert name == "qgemm_mxfp4_act"
    bp = u8(qg.qgemm_prepack_bytes(4, K, N))
    ws8 = u8(qg.qgemm_act_workspace_bytes("fp8", M, K))
    name = calls_for_shapes(lambda out: qg.qgemm_fp8_act(a, bp, scalar, N, workspace=ws8,
                                                         out=out),
                            (M, N), BAD, torch.bfloat16, rec)
    assert name == "qgemm_fp8_act"


def test_weight_only_grouped_nvfp4_out_shape_checked_before_launch(fake):
    rec, scalar = fake
    x = torch.zeros((M, K), dtype=torch.float16)
    s = torch.zeros(N, dtype=torch.float16)
    for fmt, fn in ((1, qg.qgemm_w4a16), (2, qg.qgemm_w8a16)):
        wp = u8(qg.qgemm_prepack_bytes(fmt, K, N))
        name = calls_for_shapes(lambda out: fn(x, wp, s, N, out=out), (M, N), BAD,
                                torch.float16, rec)
        assert name == fn.__name__
    for fmt, fn in ((5, qg.qgemm_w4a16_grouped), (6, qg.qgemm_w8a16_grouped)):
        wp = u8(qg.qgemm_prepack_grouped_bytes(fmt, K, N, 32))
        name = calls_for_shapes(lambda out: fn(x, wp, N, 32, out=out), (M, N), BAD,
                                torch.float16, rec)
        assert name == fn.__name__
    wp = u8(qg.qgemm_prepack_bytes(7, K, N))
    name = calls_for_shapes(lambda out: qg.qgemm_nvfp4(x, wp, scalar, N, out=out), (M, N), BAD,
                            torch.float16, rec)
    assert name == "qgemm_nvfp4"


def test_wrong_output_dtype_rejected(fake):
    rec, scalar = fake
    bp = u8(qg.qgemm_prepack_bytes(4, K, N))
    with pytest.raises(TypeError):
        qg.qgemm_fp8(u8(M, K), bp, scalar, scalar, N, out=torch.zeros((M, N), dtype=torch.float16))
    assert rec.calls == []
