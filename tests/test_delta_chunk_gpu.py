"""Gated delta rule forward, GDN chunk form (rglru_delta_chunk_fwd), through the C ABI.

Element by element against the float64 oracle (its token recurrence, which
its chunk form matches to rounding) on the same stored inputs: one chunk,
several chunks with a ragged tail, a single token, grouped key heads, both
key widths (64, 128), value widths of one to eight 32-column tiles, a
nonzero initial state, the value-first state; zero tokens (the initial state
comes back bitwise); sampled heads at the full prefill workload (B=4,
T=2048, 16 heads of 128 x 128); run-to-run determinism; the restrictions.

Tolerance. The dense products take bf16 operands: T, W, U~, the corrected
writes U, the masked Q K^T and the state's operand copy are each rounded to
bf16 (relative 2^-9) where they enter an MFMA, with float32 accumulation.
An output element sums Dk + 64 such products whose terms are of the size of
the state and the writes, so its error is a few times 2^-9 of those
magnitudes (measured: at most 2.5e-3 of max(1, |ref|) over these cases);
the bound is 2^-7 of max(1, |ref|) for outputs. The float32 state takes one
bf16-rounded update per chunk (U and the decayed k), measured at most 4.7e-3:
bound 2^-6.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from synth import delta as sd
from _helpers import host64

pytestmark = pytest.mark.gpu

O_TOL = 2.0 ** -7
S_TOL = 2.0 ** -6


@pytest.fixture(autouse=True)
def _announce(request):
    sys.__stderr__.write(f"\n[gpu-case] {request.node.nodeid}\n")
    sys.__stderr__.flush()
    yield


def _dev(stored):
    return torch.from_numpy(stored.raw.copy()).cuda().view(torch.bfloat16)


def _f32(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def _run(glr, inp, v_first=False, scale=None, fn="chunk"):
    h0 = inp.h0
    if h0 is not None and v_first:
        h0 = h0.transpose(0, 1, 3, 2)
    f = glr.rglru_delta_chunk_fwd if fn == "chunk" else glr.rglru_delta_rule_fwd
    cu = None if inp.cu is None else torch.from_numpy(inp.cu).cuda()
    o, s = f(_dev(inp.q), _dev(inp.k), _dev(inp.v), _f32(inp.g), _f32(inp.beta), scale=scale,
             initial_state=_f32(h0), cu_seqlens=cu, state_v_first=v_first)
    torch.cuda.synchronize()
    s = host64(s)
    if v_first:
        s = s.transpose(0, 1, 3, 2)
    return host64(o), s


def _ref(inp, scale=None):
    return oracle.recurrent_delta_rule(inp.q.value, inp.k.value, inp.v.value, inp.g.astype(np.float64),
                                       inp.beta.astype(np.float64), scale=scale, initial_state=inp.h0,
                                       cu_seqlens=inp.cu)


def _err(got, ref):
    return float(np.max(np.abs(got - ref) / np.maximum(1.0, np.abs(ref)))) if ref.size else 0.0


def _check(got, ref, label=""):
    eo, es = _err(got[0], ref[0]), _err(got[1], ref[1])
    sys.__stderr__.write(f"[chunk-err] {label} o {eo:.3e} state {es:.3e}\n")
    assert eo <= O_TOL and es <= S_TOL, f"{label} o err {eo:.3g} (tol {O_TOL}), state err {es:.3g} (tol {S_TOL})"


BASE = sd.DELTA_WORKLOADS[10]

CASES = [
    # (B, T, Hk, Hv, Dk, Dv, h0)
    (1, 64, 1, 1, 128, 128, False),   # exactly one chunk
    (2, 100, 1, 2, 64, 32, True),     # two chunks, ragged tail, grouped heads
    (2, 300, 2, 4, 128, 64, True),    # five chunks
    (1, 1, 1, 1, 128, 256, True),     # one token, eight column tiles
    (3, 129, 1, 1, 64, 96, False),    # three chunks, the last with one token
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}T{}Hk{}Hv{}Dk{}Dv{}{}".format(*c[:6], "-h0" if c[6] else ""))
def test_against_oracle(gpu_lib, case):
    B, T, Hk, Hv, Dk, Dv, h0 = case
    wl = BASE.resized(wid=30, batch=B, length=T, k_heads=Hk, v_heads=Hv, k_dim=Dk, v_dim=Dv, h0=h0)
    inp = sd.make_delta_inputs(wl)
    _check(_run(gpu_lib, inp), _ref(inp), str(case))


def test_value_first_state_and_scale(gpu_lib):
    wl = BASE.resized(wid=31, batch=2, length=150, k_heads=1, v_heads=2, k_dim=128, v_dim=64, h0=True)
    inp = sd.make_delta_inputs(wl)
    _check(_run(gpu_lib, inp, v_first=True, scale=0.29), _ref(inp, scale=0.29), "v_first")


@pytest.mark.parametrize("Dk", [64, 128])
def test_packed_sequences(gpu_lib, Dk):
    lens = [0, 1, 17, 64, 65, 130, 0, 5]
    wl = BASE.resized(wid=34, k_heads=1, v_heads=2, k_dim=Dk, v_dim=64, h0=True)
    inp = sd.make_delta_inputs(wl, lengths=lens)
    got = _run(gpu_lib, inp)
    _check(got, _ref(inp), f"packed Dk{Dk}")
    for n in (0, 6):   # empty sequences return their initial state bitwise
        np.testing.assert_array_equal(got[1][n], inp.h0[n].astype(np.float64))
    # each sequence alone, as a one-row call, gives the same bits
    cu = inp.cu
    for n in range(len(lens)):
        a, b = int(cu[n]), int(cu[n + 1])
        if b == a:
            continue
        one = sd.DeltaInputs(wl.resized(batch=1, length=b - a),
                             *(sd.Stored(st.io, st.raw[:, a:b].copy(), st.value[:, a:b]) for st in (inp.q, inp.k, inp.v)),
                             inp.g[:, a:b].copy(), inp.beta[:, a:b].copy(), inp.h0[n:n + 1].copy())
        o1, s1 = _run(gpu_lib, one)
        np.testing.assert_array_equal(o1[0], got[0][0, a:b])
        np.testing.assert_array_equal(s1[0], got[1][n])


def test_packed_geometric_lengths(gpu_lib):
    lens = sd.seq_lengths(24, 100.0, empty_p=0.1)
    wl = BASE.resized(wid=35, k_heads=2, v_heads=4, h0=True)
    inp = sd.make_delta_inputs(wl, lengths=lens)
    _check(_run(gpu_lib, inp), _ref(inp), "packed geometric")


def test_packed_all_empty(gpu_lib):
    wl = BASE.resized(wid=36, k_heads=1, v_heads=2, k_dim=64, v_dim=32, h0=True)
    inp = sd.make_delta_inputs(wl, lengths=[0, 0, 0])
    o, s = _run(gpu_lib, inp)
    assert o.shape == (1, 0, 2, 32)
    np.testing.assert_array_equal(s, inp.h0.astype(np.float64))


@pytest.mark.parametrize("with_h0", [False, True])
def test_zero_tokens(gpu_lib, with_h0):
    wl = BASE.resized(wid=32, batch=2, length=0, k_heads=1, v_heads=3, k_dim=64, v_dim=64, h0=with_h0)
    inp = sd.make_delta_inputs(wl)
    o, s = _run(gpu_lib, inp)
    assert o.shape == (2, 0, 3, 64)
    want = inp.h0.astype(np.float64) if with_h0 else np.zeros((2, 3, 64, 64))
    np.testing.assert_array_equal(s, want)


def test_full_prefill_sampled_and_against_token_recurrence(gpu_lib):
    """B=4, T=2048, Hk=Hv=16, Dk=Dv=128 bf16: sampled (row, head) pairs against the oracle over all
    2048 tokens, and every output against the float32 token-recurrent kernel."""
    inp = sd.make_delta_inputs(BASE)
    o, s = _run(gpu_lib, inp)
    for b, h in ((0, 0), (1, 5), (2, 15), (3, 10)):
        sl = lambda st: st.value[b:b + 1, :, h:h + 1]
        ro, rs = oracle.recurrent_delta_rule(sl(inp.q), sl(inp.k), sl(inp.v),
                                             inp.g[b:b + 1, :, h:h + 1].astype(np.float64),
                                             inp.beta[b:b + 1, :, h:h + 1].astype(np.float64))
        _check((o[b, :, h], s[b, h]), (ro[0, :, 0], rs[0, 0]), f"full b{b} h{h}")
    ro, rs = _run(gpu_lib, inp, fn="recurrent")
    _check((o, s), (ro, rs), "full vs token recurrence")


def test_run_to_run_bitwise(gpu_lib):
    wl = BASE.resized(wid=33, batch=2, length=200, k_heads=1, v_heads=2, k_dim=128, v_dim=128, h0=True)
    inp = sd.make_delta_inputs(wl)
    a, b = _run(gpu_lib, inp), _run(gpu_lib, inp)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_unsupported(gpu_lib):
    dev = torch.device("cuda")
    def mk(Dk, Dv, dt=torch.bfloat16):
        q = torch.zeros(1, 4, 1, Dk, dtype=dt, device=dev)
        v = torch.zeros(1, 4, 1, Dv, dtype=dt, device=dev)
        g = torch.zeros(1, 4, 1, device=dev)
        return q, q.clone(), v, g, g.clone()
    for args in (mk(96, 64), mk(128, 48), mk(128, 288), mk(64, 64, torch.float32)):
        with pytest.raises(gpu_lib.RglruError) as e:
            gpu_lib.rglru_delta_chunk_fwd(*args)
        assert e.value.status == 4
