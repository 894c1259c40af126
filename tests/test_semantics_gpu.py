"""Bit-exact and structural properties of the HIP path: reset isolation, determinism,
sequence continuation, the workspace contract and argument validation on the device."""
import sys

import numpy as np
import pytest
import torch

import synth
from _helpers import DevInputs, compare, host64, run_gpu, run_oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    sys.__stderr__.write(f"\n[gpu-case] {request.node.nodeid}\n")
    sys.__stderr__.flush()
    yield


def _inputs(B=2, L=300, W=256, doc=40.0, variant=0):
    wl = synth.dataclasses.replace(synth.WORKLOADS[2].resized(batch=B, length=L, width=W), doc_mean=doc)
    return synth.make_inputs(wl, variant=variant, with_dh_last=True)


@pytest.mark.parametrize("chunk", [8, 64, 256])
def test_perturbation_before_reset_leaves_later_state_bitwise(gpu_lib, chunk):
    inp = _inputs()
    d = DevInputs(inp)
    a = run_gpu(gpu_lib, d, chunk=chunk)
    reset = inp.reset
    b, first = 0, int(np.flatnonzero(reset[0])[1])   # second reset of row 0
    d2 = DevInputs(inp)
    d2.x[b, :first] = torch.randn_like(d2.x[b, :first].float()).to(d2.x.dtype)
    d2.gx[b, : first - 1] = 7.0
    d2.ga[b, : first - 1] = -3.0
    d2.h0[b] = 100.0
    c = run_gpu(gpu_lib, d2, chunk=chunk)
    assert torch.equal(a["h"][b, first:], c["h"][b, first:])
    assert torch.equal(a["h"][1 - b], c["h"][1 - b])


@pytest.mark.parametrize("chunk", [8, 64])
def test_nonfinite_before_reset_does_not_cross(gpu_lib, chunk):
    inp = _inputs()
    d = DevInputs(inp)
    a = run_gpu(gpu_lib, d, chunk=chunk, want_bwd=False)
    reset = inp.reset
    first = int(np.flatnonzero(reset[0])[1])
    d.x[0, first - 3, 5] = float("nan")
    d.ga[0, first - 2, 7] = float("inf")
    d.h0[0, 9] = float("nan")
    c = run_gpu(gpu_lib, d, chunk=chunk, want_bwd=False)
    assert torch.equal(a["h"][0, first:], c["h"][0, first:])
    assert torch.isnan(c["h"][0, first - 3, 5].float())


def test_dgate_a_exactly_zero_on_reset_tokens(gpu_lib):
    inp = _inputs()
    g = run_gpu(gpu_lib, DevInputs(inp), chunk=32)
    mask = torch.from_numpy(inp.reset.astype(bool)).cuda()
    assert torch.all(g["dga"][mask] == 0)


def test_gradients_before_reset_ignore_later_dh(gpu_lib):
    inp = _inputs()
    d = DevInputs(inp)
    a = run_gpu(gpu_lib, d, chunk=16)
    first = int(np.flatnonzero(inp.reset[0])[1])
    d.dh[0, first:] = (d.dh[0, first:].float() * -2.0 + 0.5).to(d.dh.dtype)
    d.dh_last[0] = 42.0
    c = run_gpu(gpu_lib, d, chunk=16)
    for k in ("dx", "dgx", "dga"):
        assert torch.equal(a[k][0, :first], c[k][0, :first])
    assert torch.equal(a["dh0"][0], c["dh0"][0])


@pytest.mark.parametrize("chunk", [8, 64, 256])
def test_bitwise_deterministic(gpu_lib, chunk):
    inp = _inputs(B=2, L=1000, W=512)
    d = DevInputs(inp)
    ref = run_gpu(gpu_lib, d, chunk=chunk)
    for _ in range(20):
        g = run_gpu(gpu_lib, d, chunk=chunk)
        for k in ref:
            assert torch.equal(ref[k], g[k]), k


def test_sequence_continuation(gpu_lib):
    """Running [0, L1) then [L1, L) with h0 = h_last matches the full run."""
    inp = _inputs(B=2, L=400, W=256)
    d = DevInputs(inp)
    full = run_gpu(gpu_lib, d, chunk=32, want_bwd=False)
    L1 = 173
    h1, hl1, _ = gpu_lib.rglru_fwd(d.x[:, :L1].contiguous(), d.gx[:, :L1].contiguous(), d.ga[:, :L1].contiguous(),
                                   d.lam, d.reset[:, :L1].contiguous(), d.h0, chunk=32)
    h2, hl2, _ = gpu_lib.rglru_fwd(d.x[:, L1:].contiguous(), d.gx[:, L1:].contiguous(), d.ga[:, L1:].contiguous(),
                                   d.lam, d.reset[:, L1:].contiguous(), hl1, chunk=32)
    torch.cuda.synchronize()
    got = torch.cat([h1, h2], dim=1)
    ref = host64(full["h"])
    err = np.max(np.abs(host64(got) - ref) / np.maximum(1, np.abs(ref)))
    assert err <= 4e-3
    np.testing.assert_allclose(host64(hl2), host64(full["h_last"]), rtol=1e-4, atol=1e-5)


def test_shared_workspace_across_shapes_and_directions(gpu_lib):
    ws = gpu_lib.Workspace("cuda")
    cases = ((300, 256, 64), (50, 100, 8), (1000, 512, 128), (7, 64, 16))
    ws.get(max(gpu_lib.rglru_workspace_bytes(gpu_lib.make_shape(2, L, W_, torch.bfloat16, chunk))
               for L, W_, chunk in cases))
    for L, W_, chunk in cases:
        inp = _inputs(B=2, L=L, W=W_)
        d = DevInputs(inp)
        h, hl, ck = gpu_lib.rglru_fwd(d.x, d.gx, d.ga, d.lam, d.reset, d.h0, chunk=chunk, workspace=ws)
        dx, dgx, dga, dlam, dh0 = gpu_lib.rglru_bwd(d.x, d.gx, d.ga, d.lam, d.reset, ck, d.dh, d.dh_last,
                                                    chunk=chunk, workspace=ws)
        torch.cuda.synchronize()
        compare("bf16", {"h": h, "h_last": hl, "dx": dx, "dgx": dgx, "dga": dga, "dlam": dlam, "dh0": dh0},
                run_oracle(inp), label=f"L={L} W={W_}")
    assert ws.error_bits() == 0
    hdr = ws.buf[:16].cpu().numpy().view(np.uint32)
    assert hdr[0] == 0 and hdr[2] == 0          # no ticket or done count left behind
    # one call-counter step per call, except the forward of at most 8 steps
    # (L = 7 here), which runs the serial kernel: it publishes no words
    assert hdr[1] == 7


def test_call_counter_wraps_without_tag_zero(gpu_lib):
    # The forward tags its published words with the call count + 1 and the
    # backward's words carry 0 in that half, so the count must never make a
    # tag of 0. Start the count just below 2^32 and cross the wrap: every call
    # must match a fresh workspace bitwise, and the count skips 0xFFFFFFFF.
    inp = _inputs(B=2, L=700, W=256, doc=300.0)
    d = DevInputs(inp)

    def step(ws):
        h, hl, ck = gpu_lib.rglru_fwd(d.x, d.gx, d.ga, d.lam, d.reset, d.h0, chunk=64, workspace=ws)
        grads = gpu_lib.rglru_bwd(d.x, d.gx, d.ga, d.lam, d.reset, ck, d.dh, d.dh_last, chunk=64, workspace=ws)
        torch.cuda.synchronize()
        return [t.clone() for t in (h, hl) + tuple(grads) if t is not None]

    ref = step(gpu_lib.Workspace("cuda"))
    ws = gpu_lib.Workspace("cuda")
    ws.get(gpu_lib.rglru_workspace_bytes(gpu_lib.make_shape(2, 700, 256, torch.bfloat16, 64)))
    ws.buf[4:8].view(torch.int32).fill_(np.int32(np.uint32(0xFFFFFFFB).view(np.int32)))
    counts = []
    for _ in range(4):
        got = step(ws)
        assert len(got) == len(ref) == 7
        for g, r in zip(got, ref):
            assert torch.equal(g, r)
        counts.append(int(ws.buf[4:8].cpu().numpy().view(np.uint32)[0]))
    assert counts == [0xFFFFFFFD, 0, 2, 4]
    assert ws.error_bits() == 0


def test_autograd_function(gpu_lib):
    inp = _inputs(B=2, L=130, W=128)
    d = DevInputs(inp)
    x = d.x.clone().requires_grad_(True)
    gx = d.gx.clone().requires_grad_(True)
    ga = d.ga.clone().requires_grad_(True)
    lam = d.lam.clone().requires_grad_(True)
    h0 = d.h0.clone().requires_grad_(True)
    h, h_last = gpu_lib.rglru(x, gx, ga, lam, h0, d.reset, chunk=32)
    loss = (h.float() * d.dh.float()).sum() + (h_last * d.dh_last).sum()
    loss.backward()
    torch.cuda.synchronize()
    gpu = {"h": h.detach(), "h_last": h_last.detach(), "dx": x.grad, "dgx": gx.grad, "dga": ga.grad,
           "dlam": lam.grad, "dh0": h0.grad}
    compare("bf16", gpu, run_oracle(inp))


def test_invalid_arguments_write_nothing(gpu_lib):
    import ctypes
    from gated_linear_recurrence_amd import _lib
    inp = _inputs(B=1, L=16, W=64)
    d = DevInputs(inp)
    h = torch.full_like(d.x, 3.0)
    with pytest.raises(gpu_lib.RglruError, match="INVALID"):
        gpu_lib.rglru_fwd(d.x, d.gx, d.ga, d.lam, chunk=24, h=h)
    lib = _lib.load()
    shape = gpu_lib.make_shape(1, 16, 64, torch.bfloat16)
    ws = torch.zeros(gpu_lib.rglru_workspace_bytes(shape), dtype=torch.uint8, device="cuda")
    vp = ctypes.c_void_p
    st = lib.rglru_fwd(ctypes.byref(shape), vp(d.x.data_ptr() + 1), vp(d.gx.data_ptr()), vp(d.ga.data_ptr()),
                       vp(d.lam.data_ptr()), None, None, vp(h.data_ptr()), None, None, vp(ws.data_ptr()),
                       ws.numel(), None)
    assert st == 2   # RGLRU_ERR_MISALIGNED
    st = lib.rglru_fwd(ctypes.byref(shape), vp(d.x.data_ptr()), vp(d.gx.data_ptr()), vp(d.ga.data_ptr()),
                       vp(d.lam.data_ptr()), None, None, vp(h.data_ptr()), None, None, vp(ws.data_ptr()),
                       16, None)
    assert st == 3   # RGLRU_ERR_WORKSPACE_TOO_SMALL
    torch.cuda.synchronize()
    assert torch.all(h.float() == 3.0)
