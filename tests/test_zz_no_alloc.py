"""The allocation-free forward (rglru_fwd_scratch) against rglru_fwd with a workspace.

Both run the same kernels, so the outputs must agree bitwise; two calls in a
row on the shared static workspace, the second one smaller, and a shape too
large for it, which must be refused with nothing written.
"""
import ctypes
import sys

import numpy as np
import pytest
import torch

import synth
from _helpers import DevInputs

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    sys.__stderr__.write(f"\n[gpu-case] {request.node.nodeid}\n")
    sys.__stderr__.flush()
    yield


def _inputs(B, L, W, io, doc, variant):
    wl = synth.dataclasses.replace(synth.WORKLOADS[2].resized(batch=B, length=L, width=W), io=io, doc_mean=doc)
    return DevInputs(synth.make_inputs(wl, variant=variant))


def _scratch_call(lib, d, chunk, h, h_last, ckpt):
    from gated_linear_recurrence_amd import ops
    B, L, W = d.x.shape
    shape = ops.make_shape(B, L, W, d.x.dtype, chunk)
    vp = ctypes.c_void_p

    def ptr(t):
        return None if t is None else vp(t.data_ptr())

    stream = vp(torch.cuda.current_stream().cuda_stream)
    return lib.rglru_fwd_scratch(ctypes.byref(shape), ptr(d.x), ptr(d.gx), ptr(d.ga), ptr(d.lam), ptr(d.reset),
                                 ptr(d.h0), ptr(h), ptr(h_last), ptr(ckpt), stream)


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_scratch_forward_matches_workspace_forward_twice(gpu_lib, io):
    from gated_linear_recurrence_amd import _lib
    lib = _lib.load()
    # the second call is smaller than the first: the shared array keeps the
    # first call's words, which must not leak into the second
    for B, L, W, chunk, doc, variant in ((3, 1500, 640, 0, 200.0, 1), (2, 333, 130, 32, 40.0, 2)):
        d = _inputs(B, L, W, io, doc, variant)
        ref_h, ref_hl, ref_ck = gpu_lib.rglru_fwd(d.x, d.gx, d.ga, d.lam, d.reset, d.h0, chunk=chunk,
                                                  workspace=gpu_lib.Workspace("cuda"))
        h = torch.full_like(ref_h, 7.0)
        h_last = torch.full_like(ref_hl, 7.0)
        ckpt = torch.full_like(ref_ck, 7.0)
        st = _scratch_call(lib, d, chunk, h, h_last, ckpt)
        torch.cuda.synchronize()
        assert st == 0, lib.rglru_status_string(st)
        assert torch.equal(h, ref_h), (B, L, W, io)
        assert torch.equal(h_last, ref_hl), (B, L, W, io)
        assert torch.equal(ckpt, ref_ck), (B, L, W, io)


def test_scratch_forward_binding(gpu_lib):
    d = _inputs(2, 700, 256, "bf16", 100.0, 3)
    ref = gpu_lib.rglru_fwd(d.x, d.gx, d.ga, d.lam, d.reset, d.h0)
    h = torch.empty_like(ref[0])
    hl = torch.empty_like(ref[1])
    ck = torch.empty_like(ref[2])
    got = gpu_lib.rglru_fwd_scratch(d.x, d.gx, d.ga, d.lam, d.reset, d.h0, h=h, h_last=hl, ckpt=ck)
    torch.cuda.synchronize()
    for g, r in zip(got, ref):
        assert torch.equal(g, r)


def test_scratch_forward_refuses_a_shape_beyond_its_array(gpu_lib):
    from gated_linear_recurrence_amd import _lib, ops
    lib = _lib.load()
    big = ops.make_shape(1, 65536, 4096, torch.bfloat16)
    assert lib.rglru_fwd_workspace_bytes(ctypes.byref(big)) > _lib.RGLRU_SCRATCH_BYTES
    # small real buffers: the call is refused on the shape alone and must not
    # touch any of them
    d = _inputs(1, 16, 64, "bf16", None, 0)
    h = torch.full_like(d.x, 3.0)
    vp = ctypes.c_void_p
    st = lib.rglru_fwd_scratch(ctypes.byref(big), vp(d.x.data_ptr()), vp(d.gx.data_ptr()), vp(d.ga.data_ptr()),
                               vp(d.lam.data_ptr()), None, None, vp(h.data_ptr()), None, None,
                               vp(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == 6   # RGLRU_ERR_SCRATCH_TOO_SMALL
    assert b"RGLRU_SCRATCH_BYTES" in lib.rglru_status_string(st)
    assert torch.all(h.float() == 3.0)
    with pytest.raises(gpu_lib.RglruError, match="SCRATCH_TOO_SMALL"):
        _lib.check(st, "rglru_fwd_scratch")
