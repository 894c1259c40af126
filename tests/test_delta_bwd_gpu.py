"""Gated delta rule backward (token form, rglru_delta_rule_bwd) through the C ABI.

Every gradient (dq, dk, dv, dg, dbeta, dh0) element by element against the
float64 oracle's reverse pass on the same stored inputs and output
gradients: GDN and KDA, float32 and bf16 io, both key tilings (Dk <= 64,
<= 128), value widths with a partial column block, lengths spanning several
16-token chunks with a ragged tail, grouped key heads (dq and dk sum over a
key head's value heads), the value-first state, packed sequences with empty
and one-token members; run-to-run bitwise equality (the column sums run in a
fixed order); and sampled heads at the full prefill workload.

Tolerances, elementwise |got - ref| <= tol * max(1, max |ref| of that
gradient): float32 arithmetic throughout, each gradient a sum of per-token
terms over Dk rows or Dv columns, measured below 7e-7 of the largest value;
bound 1e-5 for float32 outputs. bf16 io rounds dq, dk and dv once more
(2^-9 relative): bound 4e-3 for those.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from synth import delta as sd
from _helpers import host64

pytestmark = pytest.mark.gpu

TOL = 1e-5
TOL_BF16_OUT = 4e-3


@pytest.fixture(autouse=True)
def _announce(request):
    sys.__stderr__.write(f"\n[gpu-case] {request.node.nodeid}\n")
    sys.__stderr__.flush()
    yield


def _dev(stored):
    t = torch.from_numpy(stored.raw.copy()).cuda()
    return t.view(torch.bfloat16) if stored.io == "bf16" else t


def _f32(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def _grads(inp, seed, v_first=False):
    rng = np.random.default_rng(seed)
    B, T, Hv, Dv = inp.v.shape
    do = sd.store(rng.standard_normal((B, T, Hv, Dv)), inp.wl.io)
    n = B if inp.cu is None else len(inp.cu) - 1
    dhl = rng.standard_normal((n, Hv, inp.wl.k_dim, Dv)).astype(np.float32)
    return do, dhl


def _run(glr, inp, do, dhl, v_first=False):
    h0, dh = inp.h0, dhl
    if v_first:
        h0 = None if h0 is None else h0.transpose(0, 1, 3, 2)
        dh = dh.transpose(0, 1, 3, 2)
    cu = None if inp.cu is None else torch.from_numpy(inp.cu).cuda()
    q, k, v, g, b = _dev(inp.q), _dev(inp.k), _dev(inp.v), _f32(inp.g), _f32(inp.beta)
    _, _, ck = glr.rglru_delta_rule_fwd(q, k, v, g, b, initial_state=_f32(h0), cu_seqlens=cu, state_v_first=v_first,
                                        training=True)
    out = glr.rglru_delta_rule_bwd(q, k, v, g, b, ck, _dev(do), _f32(dh), cu_seqlens=cu, state_v_first=v_first)
    torch.cuda.synchronize()
    out = [host64(x) for x in out]
    if v_first:
        out[5] = out[5].transpose(0, 1, 3, 2)
    return out


def _ref(inp, do, dhl):
    return oracle.recurrent_delta_rule_backward(inp.q.value, inp.k.value, inp.v.value, inp.g.astype(np.float64),
                                                inp.beta.astype(np.float64), do.value, dhl.astype(np.float64),
                                                initial_state=inp.h0, cu_seqlens=inp.cu)


NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dh0")


def _check(inp, got, ref, label):
    errs = {}
    for i, (nm, a, b) in enumerate(zip(NAMES, got, ref)):
        e = float(np.max(np.abs(a - b)) / max(1.0, float(np.max(np.abs(b))))) if b.size else 0.0
        errs[nm] = e
    sys.__stderr__.write(f"[bwd-err] {label} " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()) + "\n")
    for i, nm in enumerate(NAMES):
        tol = TOL_BF16_OUT if (inp.wl.io == "bf16" and i < 3) else TOL
        assert errs[nm] <= tol, f"{label}: {nm} error {errs[nm]:.3g} (tol {tol}); all {errs}"


BASE = sd.DELTA_WORKLOADS[10]

CASES = [
    # (B, T, Hk, Hv, Dk, Dv, io, kda, h0)
    (2, 37, 1, 2, 64, 40, "f32", False, True),
    (2, 37, 1, 2, 64, 40, "bf16", True, True),
    (1, 50, 2, 4, 128, 136, "f32", True, False),
    (1, 33, 1, 1, 128, 128, "bf16", False, True),
    (3, 16, 1, 1, 8, 8, "f32", True, True),
    (2, 3, 1, 2, 64, 40, "f32", True, True),        # the checkpoint of a short (4-token chunk) forward
    (1, 4, 1, 1, 128, 128, "bf16", False, True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}T{}Hk{}Hv{}Dk{}Dv{}-{}-{}{}".format(
    c[0], c[1], c[2], c[3], c[4], c[5], c[6], "kda" if c[7] else "gdn", "-h0" if c[8] else ""))
def test_against_oracle(gpu_lib, case):
    B, T, Hk, Hv, Dk, Dv, io, kda, h0 = case
    wl = BASE.resized(wid=40, batch=B, length=T, k_heads=Hk, v_heads=Hv, k_dim=Dk, v_dim=Dv, io=io, kda=kda, h0=h0)
    inp = sd.make_delta_inputs(wl)
    do, dhl = _grads(inp, 1)
    _check(inp, _run(gpu_lib, inp, do, dhl), _ref(inp, do, dhl), str(case))


@pytest.mark.parametrize("kda", [False, True])
def test_value_first_state(gpu_lib, kda):
    wl = BASE.resized(wid=41, batch=2, length=20, k_heads=1, v_heads=1, k_dim=64, v_dim=16, io="f32", kda=kda,
                      h0=True)
    inp = sd.make_delta_inputs(wl)
    do, dhl = _grads(inp, 2)
    _check(inp, _run(gpu_lib, inp, do, dhl, v_first=True), _ref(inp, do, dhl), "v_first")


@pytest.mark.parametrize("kda", [False, True])
def test_packed_sequences(gpu_lib, kda):
    lens = [0, 1, 17, 16, 33, 0, 5]
    wl = BASE.resized(wid=42, k_heads=1, v_heads=2, k_dim=64, v_dim=32, io="f32", kda=kda, h0=True)
    inp = sd.make_delta_inputs(wl, lengths=lens)
    do, dhl = _grads(inp, 3)
    got = _run(gpu_lib, inp, do, dhl)
    _check(inp, got, _ref(inp, do, dhl), "packed")
    # empty sequences pass the final state's gradient straight to dh0
    for n in (0, 5):
        np.testing.assert_array_equal(got[5][n], dhl[n].astype(np.float64))


def test_run_to_run_bitwise(gpu_lib):
    wl = BASE.resized(wid=43, batch=2, length=45, k_heads=1, v_heads=2, k_dim=128, v_dim=64, kda=True, h0=True)
    inp = sd.make_delta_inputs(wl)
    do, dhl = _grads(inp, 4)
    a = _run(gpu_lib, inp, do, dhl)
    b = _run(gpu_lib, inp, do, dhl)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_full_prefill_sampled(gpu_lib):
    """B=4, T=2048, 16 heads of 128 x 128, bf16, GDN: sampled (row, head) pairs over all 2048 tokens."""
    inp = sd.make_delta_inputs(BASE)
    do, dhl = _grads(inp, 5)
    got = _run(gpu_lib, inp, do, dhl)
    for b, h in ((0, 3), (3, 12)):
        sl = lambda a: a[b:b + 1, :, h:h + 1]
        ref = oracle.recurrent_delta_rule_backward(sl(inp.q.value), sl(inp.k.value), sl(inp.v.value),
                                                   sl(inp.g).astype(np.float64), sl(inp.beta).astype(np.float64),
                                                   sl(do.value), dhl[b:b + 1, h:h + 1].astype(np.float64))
        mine = [got[0][b:b + 1, :, h:h + 1], got[1][b:b + 1, :, h:h + 1], got[2][b:b + 1, :, h:h + 1],
                got[3][b:b + 1, :, h:h + 1], got[4][b:b + 1, :, h:h + 1], got[5][b:b + 1, h:h + 1]]
        _check(inp, mine, ref, f"full b{b} h{h}")
