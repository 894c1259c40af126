"""The forward with both gate projections computed inside it.

Bitwise against the two-call path (projection, then the scan with 64-step
tiles on its logits), against the float64 oracle end to end, and its
refusals of shapes it does not run.
"""
import ctypes
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from _helpers import OUT_TOL, DevInputs, host64, out_err, run_oracle, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    sys.__stderr__.write(f"\n[gpu-case] {request.node.nodeid}\n")
    sys.__stderr__.flush()
    yield


def _two_call(glr, d, wx, bx, wa, ba, B, L, W):
    gx, ga = glr.rglru_blockdiag_gate_proj_fwd(d.x.view(B * L, W), wx, bx, wa, ba)
    h, hl, ck = glr.rglru_fwd(d.x, gx.view(B, L, W), ga.view(B, L, W), d.lam, d.reset, d.h0, chunk=64)
    return gx.view(B, L, W), ga.view(B, L, W), h, hl, ck


@pytest.mark.parametrize("wid,B,L", [(5, 2, 300), (4, 2, 777), (4, 1, 9), (5, 3, 64), (4, 2, 2048 + 13)])
def test_fused_forward_is_the_two_call_path_bitwise(gpu_lib, wid, B, L):
    wl = synth.WORKLOADS[wid].resized(batch=B, length=L)
    inp = synth.make_inputs(wl)
    d = DevInputs(inp)
    wx, wa, bx, ba = (to_dev(s) for s in (inp.wx, inp.wa, inp.bx, inp.ba))
    ref = _two_call(gpu_lib, d, wx, bx, wa, ba, B, L, wl.width)
    h, hl, ck, gx, ga = gpu_lib.rglru_blockdiag_fused_fwd(d.x, wx, bx, wa, ba, d.lam, d.reset, d.h0,
                                                          want_gates=True)
    torch.cuda.synchronize()
    for name, got, want in (("gate_x", gx, ref[0]), ("gate_a", ga, ref[1]), ("h", h, ref[2]),
                            ("h_last", hl, ref[3]), ("ckpt", ck, ref[4])):
        assert torch.equal(got, want), f"{name} differs (workload {wid}, B={B} L={L})"


def test_fused_forward_with_nonzero_bias_and_without_gate_outputs(gpu_lib):
    wl = synth.WORKLOADS[5].resized(batch=2, length=200)
    inp = synth.make_inputs(wl)
    d = DevInputs(inp)
    wx, wa = to_dev(inp.wx), to_dev(inp.wa)
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    bx = torch.randn(wl.width, device="cuda", generator=g).to(torch.bfloat16)
    ba = torch.randn(wl.width, device="cuda", generator=g).to(torch.bfloat16)
    ref = _two_call(gpu_lib, d, wx, bx, wa, ba, 2, 200, wl.width)
    h, hl, ck, gx, ga = gpu_lib.rglru_blockdiag_fused_fwd(d.x, wx, bx, wa, ba, d.lam, d.reset, d.h0,
                                                          training=False)
    torch.cuda.synchronize()
    assert gx is None and ga is None and ck is None
    assert torch.equal(h, ref[2]) and torch.equal(hl, ref[3])


@pytest.mark.parametrize("L", [1, 5, 300])
def test_fused_forward_against_oracle(gpu_lib, L):
    # float64 projection rounded once to bf16 (as the path stores logits),
    # then the float64 scan: the single-stage output tolerance (L <= 8 runs
    # the tiled kernel here, where the two-call path takes the serial one)
    wl = synth.WORKLOADS[4].resized(batch=2, length=L)
    inp = synth.make_inputs(wl)
    B, L, W = wl.batch, wl.length, wl.width
    d = DevInputs(inp)
    wx, wa, bx, ba = (to_dev(s) for s in (inp.wx, inp.wa, inp.bx, inp.ba))
    h, hl, _, gx, ga = gpu_lib.rglru_blockdiag_fused_fwd(d.x, wx, bx, wa, ba, d.lam, d.reset, d.h0,
                                                         want_gates=True)
    torch.cuda.synchronize()
    xv = inp.x.value.reshape(B * L, W)
    rgx = oracle.blockdiag_proj_forward(xv, inp.wx.value, inp.bx.value)
    rga = oracle.blockdiag_proj_forward(xv, inp.wa.value, inp.ba.value)
    gin = synth.Inputs(wl, inp.x, synth.Stored("bf16", None, synth.store(rgx, "bf16").value.reshape(B, L, W)),
                       synth.Stored("bf16", None, synth.store(rga, "bf16").value.reshape(B, L, W)), inp.lam,
                       inp.dh, inp.reset, inp.h0, inp.dh_last)
    ref = run_oracle(gin, want_bwd=False)
    err = out_err(host64(h), ref["h"])
    assert err <= OUT_TOL["bf16"], err
    assert out_err(host64(hl), ref["h_last"]) <= OUT_TOL["bf16"]


def test_fused_forward_full_size_pages_scope(gpu_lib):
    # the pages' measured scope at their shape: bitwise against the two calls
    wl = synth.WORKLOADS[5]
    inp = synth.make_inputs(wl)
    B, L, W = wl.batch, wl.length, wl.width
    d = DevInputs(inp)
    wx, wa, bx, ba = (to_dev(s) for s in (inp.wx, inp.wa, inp.bx, inp.ba))
    ref = _two_call(gpu_lib, d, wx, bx, wa, ba, B, L, W)
    h, hl, ck, gx, ga = gpu_lib.rglru_blockdiag_fused_fwd(d.x, wx, bx, wa, ba, d.lam, d.reset, d.h0,
                                                          want_gates=True)
    torch.cuda.synchronize()
    assert torch.equal(gx, ref[0]) and torch.equal(ga, ref[1])
    assert torch.equal(h, ref[2]) and torch.equal(ck, ref[4])


def test_fused_forward_refuses_unsupported_shapes(gpu_lib):
    from gated_linear_recurrence_amd import _lib, ops
    lib = _lib.load()
    wl = synth.WORKLOADS[5].resized(batch=1, length=64)
    inp = synth.make_inputs(wl)
    d = DevInputs(inp)
    wx, wa = to_dev(inp.wx), to_dev(inp.wa)
    h = torch.full_like(d.x, 3.0)
    ws = torch.zeros(1 << 22, dtype=torch.uint8, device="cuda")
    vp = ctypes.c_void_p
    for shape in (ops.make_shape(1, 64, 2048, torch.bfloat16, 32),     # chunk other than 0 or 64
                  ops.make_shape(1, 64, 2048 - 64, torch.bfloat16),    # width not a multiple of 256
                  ops.make_shape(1, 64, 2048, torch.float32)):         # float32 io
        st = lib.rglru_blockdiag_fused_fwd(ctypes.byref(shape), vp(d.x.data_ptr()), vp(wx.data_ptr()), None,
                                           vp(wa.data_ptr()), None, vp(d.lam.data_ptr()), None, None,
                                           vp(h.data_ptr()), None, None, None, None, vp(ws.data_ptr()),
                                           ws.numel(), vp(torch.cuda.current_stream().cuda_stream))
        assert st == 4   # RGLRU_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.all(h.float() == 3.0)
