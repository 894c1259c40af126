"""Block-diagonal gate projections on MFMA vs the float64 oracle, and the
projection feeding the scan end to end (the 8 x 4096 x 2560 workload)."""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from _helpers import DevInputs, GRAD_TOL, OUT_TOL, compare, grad_err, host64, out_err, run_oracle, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    sys.__stderr__.write(f"\n[gpu-case] {request.node.nodeid}\n")
    sys.__stderr__.flush()
    yield


def _proj_inputs(T, nb, variant=0, bias=True):
    W = nb * 256
    x = synth.normal(4, synth.T_X, (T, W), "bf16", variant)
    wx = synth.normal(4, synth.T_WX, (nb, 256, 256), "bf16", variant, scale=1 / 16)
    wa = synth.normal(4, synth.T_WA, (nb, 256, 256), "bf16", variant, scale=1 / 16)
    rng = np.random.default_rng(100 + variant)
    dgx = synth.store(rng.standard_normal((T, W)), "bf16")
    dga = synth.store(rng.standard_normal((T, W)), "bf16")
    dxi = synth.store(rng.standard_normal((T, W)), "bf16")
    bx = synth.store(rng.standard_normal(W) * 0.5 if bias else np.zeros(W), "bf16")
    ba = synth.store(rng.standard_normal(W) * 0.5 if bias else np.zeros(W), "bf16")
    return x, wx, wa, bx, ba, dgx, dga, dxi


@pytest.mark.parametrize("T,nb", [(1, 1), (37, 1), (300, 2), (1000, 3)])
def test_projection_forward_small(gpu_lib, T, nb):
    x, wx, wa, bx, ba, *_ = _proj_inputs(T, nb)
    gx, ga = gpu_lib.rglru_blockdiag_gate_proj_fwd(to_dev(x), to_dev(wx), to_dev(bx), to_dev(wa), to_dev(ba))
    torch.cuda.synchronize()
    rx = oracle.blockdiag_proj_forward(x.value, wx.value, bx.value)
    ra = oracle.blockdiag_proj_forward(x.value, wa.value, ba.value)
    assert out_err(host64(gx), rx) <= OUT_TOL["bf16"]
    assert out_err(host64(ga), ra) <= OUT_TOL["bf16"]


@pytest.mark.parametrize("T,nb,with_dx_in", [(1, 1, True), (45, 1, False), (300, 2, True), (1000, 3, True), (5000, 2, False)])
def test_projection_backward_small(gpu_lib, T, nb, with_dx_in):
    x, wx, wa, _, _, dgx, dga, dxi = _proj_inputs(T, nb)
    dx, dwx, dbx, dwa, dba = gpu_lib.rglru_blockdiag_gate_proj_bwd(
        to_dev(x), to_dev(wx), to_dev(wa), to_dev(dgx), to_dev(dga), to_dev(dxi) if with_dx_in else None)
    torch.cuda.synchronize()
    rdx_x, rdw_x, rdb_x = oracle.blockdiag_proj_backward(x.value, wx.value, dgx.value)
    rdx_a, rdw_a, rdb_a = oracle.blockdiag_proj_backward(x.value, wa.value, dga.value)
    rdx = rdx_x + rdx_a + (dxi.value if with_dx_in else 0.0)
    tol = GRAD_TOL["bf16"]
    assert grad_err(host64(dx), rdx) <= tol
    assert grad_err(host64(dwx), rdw_x) <= tol
    assert grad_err(host64(dwa), rdw_a) <= tol
    assert grad_err(host64(dbx), rdb_x) <= tol
    assert grad_err(host64(dba), rdb_a) <= tol


def test_projection_backward_in_place_dx(gpu_lib):
    x, wx, wa, _, _, dgx, dga, dxi = _proj_inputs(257, 2)
    d_in = to_dev(dxi)
    ref, *_ = gpu_lib.rglru_blockdiag_gate_proj_bwd(to_dev(x), to_dev(wx), to_dev(wa), to_dev(dgx), to_dev(dga),
                                                    d_in.clone())
    out, *_ = gpu_lib.rglru_blockdiag_gate_proj_bwd(to_dev(x), to_dev(wx), to_dev(wa), to_dev(dgx), to_dev(dga),
                                                    d_in, dx_out=d_in)
    torch.cuda.synchronize()
    assert torch.equal(ref, out)


def test_projection_full_size_sampled(gpu_lib):
    """B*L = 32768 tokens, 10 blocks: every token row of sampled blocks; dW/db on sampled blocks."""
    T, nb = 8 * 4096, 10
    x, wx, wa, bx, ba, dgx, dga, dxi = _proj_inputs(T, nb, bias=False)
    dev = {k: to_dev(v) for k, v in dict(x=x, wx=wx, wa=wa, bx=bx, ba=ba, dgx=dgx, dga=dga, dxi=dxi).items()}
    gx, ga = gpu_lib.rglru_blockdiag_gate_proj_fwd(dev["x"], dev["wx"], dev["bx"], dev["wa"], dev["ba"])
    dx, dwx, dbx, dwa, dba = gpu_lib.rglru_blockdiag_gate_proj_bwd(dev["x"], dev["wx"], dev["wa"], dev["dgx"],
                                                                   dev["dga"], dev["dxi"])
    torch.cuda.synchronize()
    for kb in (0, 4, 9):
        sl = slice(kb * 256, (kb + 1) * 256)
        xb = x.value[:, sl]
        for g, w, out in ((0, wx, gx), (1, wa, ga)):
            ref = xb @ w.value[kb]
            assert out_err(host64(out[:, sl]), ref) <= OUT_TOL["bf16"], (kb, g)
        ref_dx = dgx.value[:, sl] @ wx.value[kb].T + dga.value[:, sl] @ wa.value[kb].T + dxi.value[:, sl]
        assert grad_err(host64(dx[:, sl]), ref_dx) <= GRAD_TOL["bf16"], kb
        for dw, db, dg in ((dwx, dbx, dgx), (dwa, dba, dga)):
            assert grad_err(host64(dw[kb]), xb.T @ dg.value[:, sl]) <= GRAD_TOL["bf16"], kb
            assert grad_err(host64(db[sl]), dg.value[:, sl].sum(0)) <= GRAD_TOL["bf16"], kb


@pytest.mark.parametrize("wid", [4, 5])
def test_projection_feeding_scan_end_to_end(gpu_lib, wid):
    """Projection -> scan -> scan backward -> projection backward, against the oracle composed the same way
    (workload 4: resets and an initial state; 5: the restricted contract at width 2048)."""
    wl = synth.WORKLOADS[wid].resized(batch=2, length=300)
    inp = synth.make_inputs(wl, with_dh_last=True)
    B, L, W = wl.batch, wl.length, wl.width
    d = DevInputs(inp)
    wx, wa, bx, ba = (to_dev(s) for s in (inp.wx, inp.wa, inp.bx, inp.ba))
    x2 = d.x.view(B * L, W)
    gx, ga = gpu_lib.rglru_blockdiag_gate_proj_fwd(x2, wx, bx, wa, ba)
    h, h_last, ckpt = gpu_lib.rglru_fwd(d.x, gx.view(B, L, W), ga.view(B, L, W), d.lam, d.reset, d.h0)
    dxs, dgx, dga, dlam, dh0 = gpu_lib.rglru_bwd(d.x, gx.view(B, L, W), ga.view(B, L, W), d.lam, d.reset, ckpt,
                                                 d.dh, d.dh_last)
    dx, dwx, dbx, dwa, dba = gpu_lib.rglru_blockdiag_gate_proj_bwd(x2, wx, wa, dgx.view(B * L, W),
                                                                   dga.view(B * L, W), dxs.view(B * L, W))
    torch.cuda.synchronize()

    # stage 1: projection against float64
    xv = inp.x.value.reshape(B * L, W)
    rgx = oracle.blockdiag_proj_forward(xv, inp.wx.value, inp.bx.value)
    rga = oracle.blockdiag_proj_forward(xv, inp.wa.value, inp.ba.value)
    assert out_err(host64(gx), rgx) <= OUT_TOL["bf16"]
    assert out_err(host64(ga), rga) <= OUT_TOL["bf16"]
    # stage 2: the scan on the GPU's own bf16 logits
    gin = synth.Inputs(wl, inp.x, synth.Stored("bf16", None, host64(gx).reshape(B, L, W)),
                       synth.Stored("bf16", None, host64(ga).reshape(B, L, W)), inp.lam, inp.dh, inp.reset,
                       inp.h0, inp.dh_last)
    ref = run_oracle(gin)
    compare("bf16", {"h": h, "h_last": h_last, "dgx": dgx, "dga": dga, "dlam": dlam, "dh0": dh0}, ref)
    # stage 3: gradients through both stages (scan dx plus the projections' dx), on the GPU's own dgates
    dgxv = host64(dgx).reshape(B * L, W)
    dgav = host64(dga).reshape(B * L, W)
    rdx_x, rdw_x, rdb_x = oracle.blockdiag_proj_backward(xv, inp.wx.value, dgxv)
    rdx_a, rdw_a, rdb_a = oracle.blockdiag_proj_backward(xv, inp.wa.value, dgav)
    rdx = ref["dx"].reshape(B * L, W) + rdx_x + rdx_a
    assert grad_err(host64(dx), rdx) <= GRAD_TOL["bf16"]
    for got, want in ((dwx, rdw_x), (dwa, rdw_a), (dbx, rdb_x), (dba, rdb_a)):
        assert grad_err(host64(got), want) <= GRAD_TOL["bf16"]
    # End to end: the float64 projection, rounded once to bf16 (as the path
    # stores its logits), through the float64 scan. The GPU's logits are those
    # rounded values up to the float32 accumulation: a bf16 rounding of the
    # float32 sum can land one spacing away, and the sum itself is within
    # bs * 2^-24 * sum|x w| of the exact one (the usual bound for a float32
    # dot product of bs terms). h is then held to the single-stage output
    # tolerance.
    bs = wl.proj_block
    rq = {}
    for name, got, ref64, w, b in (("gate_x", gx, rgx, inp.wx.value, inp.bx.value),
                                   ("gate_a", ga, rga, inp.wa.value, inp.ba.value)):
        q = synth.store(ref64, "bf16").value
        g = host64(got)
        absdot = oracle.blockdiag_proj_forward(np.abs(xv), np.abs(w), None if b is None else np.abs(b))

        def spacing(v):
            return np.exp2(np.floor(np.log2(np.maximum(np.abs(v), 1e-30))) - 7)

        bound = np.maximum(spacing(q), spacing(g)) + bs * 2.0 ** -24 * absdot
        diff = g != q
        assert diff.mean() <= 1e-2, (name, diff.mean())
        assert np.all(np.abs(g - q) <= bound), (name, float(np.max(np.abs(g - q) / bound)))
        rq[name] = q.reshape(B, L, W)
    e2e_in = synth.Inputs(wl, inp.x, synth.Stored("bf16", None, rq["gate_x"]),
                          synth.Stored("bf16", None, rq["gate_a"]), inp.lam, inp.dh, inp.reset,
                          inp.h0, inp.dh_last)
    e2e = run_oracle(e2e_in, want_bwd=False)
    err = out_err(host64(h), e2e["h"])
    print(f"end-to-end h error vs bf16-rounded oracle logits: {err:.3e}")
    assert err <= OUT_TOL["bf16"]
