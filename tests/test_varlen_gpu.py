"""Packed variable-length sequences (cu_seqlens) on the HIP path.

Against the float64 oracle, each sequence as its own row, element by element;
bitwise against the one-row call where both describe the same computation;
the edge cases of the boundary: empty sequences, one-token sequences,
sequences crossing tiles, a total of at most 8 tokens (the serial kernel),
resets inside sequences, and offsets that are not valid.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from _helpers import GRAD_EL_TOL, GRAD_TOL, OUT_TOL, grad_err, host64, out_err, to_dev, to_dev_f32, to_dev_u8

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    sys.__stderr__.write(f"\n[gpu-case] {request.node.nodeid}\n")
    sys.__stderr__.flush()
    yield


class Dev:
    def __init__(self, v: synth.VarlenInputs):
        self.v = v
        self.cu = torch.from_numpy(v.cu).cuda()
        self.x, self.gx, self.ga, self.dh = (to_dev(s) for s in (v.x, v.gx, v.ga, v.dh))
        self.lam = to_dev_f32(v.lam)
        self.reset = to_dev_u8(v.reset)
        self.h0 = to_dev_f32(v.h0)
        self.dh_last = to_dev_f32(v.dh_last)


def run_gpu(glr, d, chunk=0, want_bwd=True):
    h, h_last, ckpt = glr.rglru_fwd_varlen(d.x, d.gx, d.ga, d.lam, d.cu, d.reset, d.h0, chunk=chunk)
    out = {"h": h, "h_last": h_last}
    if want_bwd:
        dx, dgx, dga, dlam, dh0 = glr.rglru_bwd_varlen(d.x, d.gx, d.ga, d.lam, d.cu, d.reset, d.h0, ckpt, d.dh,
                                                       d.dh_last, chunk=chunk)
        out.update(dx=dx, dgx=dgx, dga=dga, dlam=dlam, dh0=dh0)
    torch.cuda.synchronize()
    return out


def run_oracle(v: synth.VarlenInputs):
    h, h_last = oracle.rglru_forward_varlen(v.x.value, v.gx.value, v.ga.value, v.lam, v.cu, v.reset, v.h0)
    out = {"h": h, "h_last": h_last}
    out.update(oracle.rglru_backward_varlen(v.x.value, v.gx.value, v.ga.value, v.lam, v.dh.value, v.cu, v.reset,
                                            v.h0, v.dh_last))
    return out


def compare(io, gpu, ref, label=""):
    errs, bad = {}, {}
    errs["h"] = out_err(host64(gpu["h"]), ref["h"])
    errs["h_last"] = out_err(host64(gpu["h_last"]), ref["h_last"])
    for k in ("dx", "dgx", "dga"):
        g = host64(gpu[k])
        errs[k] = grad_err(g, ref[k])
        errs[k + " (elementwise)"] = out_err(g, ref[k])
    errs["dlam"] = grad_err(host64(gpu["dlam"]), ref["dlam"])
    errs["dh0"] = grad_err(host64(gpu["dh0"]), ref["dh0"])
    for k, e in errs.items():
        tol = (OUT_TOL if k in ("h", "h_last") else GRAD_EL_TOL if "elementwise" in k else GRAD_TOL)[io]
        if not e <= tol:
            bad[k] = (e, tol)
    assert not bad, f"{label}: {bad} (all: {errs})"


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("chunk", [0, 16])
def test_packed_sequences_against_oracle(gpu_lib, io, chunk):
    # ragged lengths from 1 token up, a few empty sequences, resets inside
    lens = synth.seq_lengths(40, 90.0, variant=1, empty_p=0.1)
    lens[3], lens[4], lens[5] = 1, 0, 1
    v = synth.make_varlen_inputs(lens, 320, io, variant=1, reset_mean=300.0)
    compare(io, run_gpu(gpu_lib, Dev(v), chunk=chunk), run_oracle(v), f"{io} chunk {chunk} T={v.cu[-1]}")


@pytest.mark.parametrize("lens", [[1], [3, 0, 2], [1, 1, 1, 1, 1, 1, 1, 1], [0, 8, 0], [5, 2]])
def test_packed_short_totals_serial_kernel(gpu_lib, lens):
    # at most 8 tokens in all: the serial kernel
    v = synth.make_varlen_inputs(lens, 130, "bf16", variant=2, reset_mean=3.0)
    compare("bf16", run_gpu(gpu_lib, Dev(v)), run_oracle(v), f"lens {lens}")


def test_packed_long_sequences_cross_many_tiles(gpu_lib):
    lens = [1, 3000, 7, 0, 2500, 129, 128, 127, 1]
    v = synth.make_varlen_inputs(lens, 256, "bf16", variant=3)
    compare("bf16", run_gpu(gpu_lib, Dev(v)), run_oracle(v), "long")


def test_packed_without_initial_states_or_final_gradients(gpu_lib):
    v = synth.make_varlen_inputs(synth.seq_lengths(25, 60.0, variant=4), 192, "bf16", variant=4,
                                 with_h0=False, with_dh_last=False)
    compare("bf16", run_gpu(gpu_lib, Dev(v)), run_oracle(v), "no h0")


def test_reset_at_every_start_is_the_one_row_call_bitwise(gpu_lib):
    # zero initial states and a reset token on every non-empty sequence's
    # first token: the packed call and the one-row call with those resets run
    # the same arithmetic
    lens = synth.seq_lengths(30, 70.0, variant=5, empty_p=0.1)
    v = synth.make_varlen_inputs(lens, 256, "bf16", variant=5, reset_mean=200.0, with_h0=False,
                                 with_dh_last=False)
    starts = np.zeros(int(v.cu[-1]), dtype=np.uint8)
    starts[v.cu[:-1][lens > 0]] = 1
    v.reset = np.maximum(v.reset, starts)
    d = Dev(v)
    got = run_gpu(gpu_lib, d)
    T, W = d.x.shape
    h, hl, ck = gpu_lib.rglru_fwd(d.x.view(1, T, W), d.gx.view(1, T, W), d.ga.view(1, T, W), d.lam,
                                  d.reset.view(1, T))
    dx, dgx, dga, dlam, _ = gpu_lib.rglru_bwd(d.x.view(1, T, W), d.gx.view(1, T, W), d.ga.view(1, T, W), d.lam,
                                              d.reset.view(1, T), ck, d.dh.view(1, T, W))
    torch.cuda.synchronize()
    assert torch.equal(got["h"], h[0])
    for name, ref in (("dx", dx), ("dgx", dgx), ("dga", dga)):
        assert torch.equal(got[name], ref[0]), name
    assert torch.equal(got["dlam"], dlam)
    ends = v.cu[1:][lens > 0] - 1
    # h_last is the float32 state, h its bf16 rounding
    np.testing.assert_allclose(host64(got["h_last"])[lens > 0], host64(h[0])[ends], rtol=4e-3, atol=4e-3)
    assert torch.all(got["h_last"][torch.from_numpy(np.flatnonzero(lens == 0)).cuda()] == 0)
    assert torch.all(got["dh0"] == 0)


def test_invalid_offsets_set_the_error_bit(gpu_lib):
    # offsets that go backwards: the call runs (every access stays in
    # bounds) and reports it in the workspace's error word
    v = synth.make_varlen_inputs([5, 7, 4], 64, "bf16", variant=6)
    d = Dev(v)
    d.cu = torch.tensor([0, 9, 5, 16], dtype=torch.int32, device="cuda")
    ws = gpu_lib.Workspace("cuda")
    gpu_lib.rglru_fwd_varlen(d.x, d.gx, d.ga, d.lam, d.cu, d.reset, d.h0, workspace=ws)
    assert ws.error_bits() & 4
    ws.clear_errors()
    assert ws.error_bits() == 0
