"""Gated delta rule forward (GDN / KDA token recurrence) on the HIP path, through the C ABI.

Element by element against the float64 oracle on the same stored inputs, at
sizes that span several 16-token chunks with a ragged tail and several
column blocks with a partial last one, for each key-dimension tiling the
library selects (Dk <= 64, <= 128, <= 256); packed sequences with empty and
one-token members; zero-token calls; one decode step; calls of at most 4
tokens per sequence, which stage 4-token chunks (every tiling, packed, the
value-first state); the value-first state;
grouped key heads (bitwise against repeated heads); run-to-run determinism;
and, at the full prefill workload (B=4, T=2048, 16 heads of 128 x 128),
sampled (batch row, head) pairs.

Tolerances, elementwise |got - ref| <= tol * max(1, |ref|): the state is
float32 on both io dtypes and each token adds two Dk-term float32 dot
products and one rank-1 write, with keys of unit length and beta < 1 so the
step is non-expansive and decays below 1 forget old rounding; 2e-5 bounds the
float32 drift (with margin) for the state and the float32 output. A bf16
output adds its own rounding, 2^-9 relative: 4e-3.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from synth import delta as sd
from _helpers import host64

pytestmark = pytest.mark.gpu

TOL = {"f32": 2e-5, "bf16": 4e-3}
STATE_TOL = 2e-5


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


def _run(glr, inp, v_first=False, scale=None):
    h0 = inp.h0
    if h0 is not None and v_first:
        h0 = h0.transpose(0, 1, 3, 2)
    cu = None if inp.cu is None else torch.from_numpy(inp.cu).cuda()
    o, s = glr.rglru_delta_rule_fwd(_dev(inp.q), _dev(inp.k), _dev(inp.v), _f32(inp.g), _f32(inp.beta),
                                    scale=scale, initial_state=_f32(h0), cu_seqlens=cu, state_v_first=v_first)
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


def _check(inp, got, ref, label=""):
    eo, es = _err(got[0], ref[0]), _err(got[1], ref[1])
    tol = TOL[inp.wl.io]
    assert eo <= tol and es <= STATE_TOL, f"{label} o err {eo:.3g} (tol {tol}), state err {es:.3g} (tol {STATE_TOL})"
    return eo, es


BASE = sd.DELTA_WORKLOADS[10]

CASES = [
    # (B, T, Hk, Hv, Dk, Dv, io, kda, h0)
    (2, 37, 1, 2, 64, 40, "bf16", False, True),     # Dk <= 64 tiling, 2 column blocks of 32, grouped heads
    (2, 50, 2, 4, 128, 136, "bf16", True, True),    # Dk <= 128 tiling, 9 column blocks of 16, last partial
    (1, 33, 1, 1, 128, 128, "f32", False, False),   # two full chunks and one token
    (1, 20, 1, 2, 256, 64, "f32", True, True),      # Dk <= 256 tiling
    (1, 21, 1, 1, 200, 24, "bf16", False, True),    # Dk not a power of two
    (3, 17, 1, 1, 8, 8, "f32", True, False),        # smallest dims
    (1, 64, 1, 1, 96, 16, "bf16", True, False),     # length an exact multiple of the chunk
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}T{}Hk{}Hv{}Dk{}Dv{}-{}-{}{}".format(
    c[0], c[1], c[2], c[3], c[4], c[5], c[6], "kda" if c[7] else "gdn", "-h0" if c[8] else ""))
def test_against_oracle(gpu_lib, case):
    B, T, Hk, Hv, Dk, Dv, io, kda, h0 = case
    wl = BASE.resized(wid=20, batch=B, length=T, k_heads=Hk, v_heads=Hv, k_dim=Dk, v_dim=Dv, io=io, kda=kda, h0=h0)
    inp = sd.make_delta_inputs(wl)
    _check(inp, _run(gpu_lib, inp), _ref(inp), str(case))


SHORT_CASES = [
    # calls of at most 4 tokens per sequence (decode-like) stage 4-token chunks
    (3, 1, 1, 2, 64, 40, "bf16", True, True),
    (2, 2, 2, 4, 128, 136, "bf16", False, True),
    (2, 4, 1, 1, 128, 128, "f32", True, False),
    (1, 3, 1, 2, 256, 64, "f32", False, True),
    (1, 4, 1, 1, 200, 24, "bf16", True, True),
    (2, 5, 1, 2, 128, 64, "bf16", False, True),     # one token past it: 16-token chunks again
]


@pytest.mark.parametrize("case", SHORT_CASES, ids=lambda c: "B{}T{}Hk{}Hv{}Dk{}Dv{}-{}-{}{}".format(
    c[0], c[1], c[2], c[3], c[4], c[5], c[6], "kda" if c[7] else "gdn", "-h0" if c[8] else ""))
def test_short_calls_against_oracle(gpu_lib, case):
    B, T, Hk, Hv, Dk, Dv, io, kda, h0 = case
    wl = BASE.resized(wid=27, batch=B, length=T, k_heads=Hk, v_heads=Hv, k_dim=Dk, v_dim=Dv, io=io, kda=kda, h0=h0)
    inp = sd.make_delta_inputs(wl)
    _check(inp, _run(gpu_lib, inp), _ref(inp), str(case))


@pytest.mark.parametrize("kda", [False, True])
def test_short_packed_and_value_first(gpu_lib, kda):
    lens = [1, 0, 2, 1]   # four tokens in all: the short chunks
    wl = BASE.resized(wid=28, k_heads=1, v_heads=2, k_dim=128, v_dim=64, kda=kda, h0=True)
    inp = sd.make_delta_inputs(wl, lengths=lens)
    got = _run(gpu_lib, inp)
    _check(inp, got, _ref(inp))
    np.testing.assert_array_equal(got[1][1], inp.h0[1].astype(np.float64))
    wl = BASE.resized(wid=29, batch=2, length=3, k_heads=1, v_heads=2, k_dim=64, v_dim=48, io="f32",
                      kda=kda, h0=True)
    inp = sd.make_delta_inputs(wl)
    _check(inp, _run(gpu_lib, inp, v_first=True), _ref(inp))


@pytest.mark.parametrize("kda", [False, True])
def test_value_first_state_and_explicit_scale(gpu_lib, kda):
    wl = BASE.resized(wid=21, batch=2, length=29, k_heads=1, v_heads=2, k_dim=128, v_dim=48, io="f32",
                      kda=kda, h0=True)
    inp = sd.make_delta_inputs(wl)
    got = _run(gpu_lib, inp, v_first=True, scale=0.37)
    _check(inp, got, _ref(inp, scale=0.37))


@pytest.mark.parametrize("kda", [False, True])
def test_packed_sequences(gpu_lib, kda):
    lens = [0, 1, 17, 16, 33, 0, 5]
    wl = BASE.resized(wid=22, k_heads=2, v_heads=2, k_dim=64, v_dim=64, kda=kda, h0=True)
    inp = sd.make_delta_inputs(wl, lengths=lens)
    got = _run(gpu_lib, inp)
    _check(inp, got, _ref(inp))
    # empty sequences carry their initial state through bitwise
    for n in (0, 5):
        np.testing.assert_array_equal(got[1][n], inp.h0[n].astype(np.float64))


def test_packed_geometric_lengths(gpu_lib):
    lens = sd.seq_lengths(24, 40.0, empty_p=0.1)
    wl = BASE.resized(wid=23, k_heads=1, v_heads=2, k_dim=128, v_dim=128, h0=True)
    inp = sd.make_delta_inputs(wl, lengths=lens)
    _check(inp, _run(gpu_lib, inp), _ref(inp))


@pytest.mark.parametrize("with_h0", [False, True])
def test_zero_tokens(gpu_lib, with_h0):
    wl = BASE.resized(wid=24, batch=3, length=0, k_heads=1, v_heads=2, k_dim=64, v_dim=32, h0=with_h0)
    inp = sd.make_delta_inputs(wl)
    o, s = _run(gpu_lib, inp)
    assert o.shape == (3, 0, 2, 32)
    want = inp.h0.astype(np.float64) if with_h0 else np.zeros((3, 2, 64, 32))
    np.testing.assert_array_equal(s, want)


def test_decode_step(gpu_lib):
    """One token of 64 sequences from a nonzero state (the serving step)."""
    inp = sd.make_delta_inputs(sd.DELTA_WORKLOADS[12])
    _check(inp, _run(gpu_lib, inp), _ref(inp), "decode")


def test_grouped_heads_bitwise_equal_repeated_heads(gpu_lib):
    wl = BASE.resized(wid=25, batch=1, length=40, k_heads=2, v_heads=6, k_dim=128, v_dim=32, kda=True)
    inp = sd.make_delta_inputs(wl)
    o1, s1 = _run(gpu_lib, inp)
    rep = lambda st: sd.Stored(st.io, np.repeat(st.raw, 3, axis=2), np.repeat(st.value, 3, axis=2))
    inp2 = sd.DeltaInputs(wl.resized(k_heads=6), rep(inp.q), rep(inp.k), inp.v, inp.g, inp.beta, inp.h0)
    o2, s2 = _run(gpu_lib, inp2)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(s1, s2)


def test_run_to_run_bitwise(gpu_lib):
    wl = BASE.resized(wid=26, batch=2, length=100, k_heads=1, v_heads=4, k_dim=128, v_dim=128, h0=True)
    inp = sd.make_delta_inputs(wl)
    a = _run(gpu_lib, inp)
    b = _run(gpu_lib, inp)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


@pytest.mark.parametrize("wid", [10, 11])
def test_full_prefill_sampled(gpu_lib, wid):
    """B=4, T=2048, Hk=Hv=16, Dk=Dv=128 bf16 in the launch the benchmark times; the oracle
    recomputes sampled (batch row, head) pairs over all 2048 tokens."""
    inp = sd.make_delta_inputs(sd.DELTA_WORKLOADS[wid])
    o, s = _run(gpu_lib, inp)
    for b, h in ((0, 0), (1, 7), (2, 15), (3, 9)):
        sl = lambda st, hh: st.value[b:b + 1, :, hh:hh + 1]
        ro, rs = oracle.recurrent_delta_rule(sl(inp.q, h), sl(inp.k, h), sl(inp.v, h),
                                             inp.g[b:b + 1, :, h:h + 1].astype(np.float64),
                                             inp.beta[b:b + 1, :, h:h + 1].astype(np.float64))
        eo, es = _err(o[b, :, h], ro[0, :, 0]), _err(s[b, h], rs[0, 0])
        assert eo <= TOL["bf16"] and es <= STATE_TOL, (b, h, eo, es)


def test_unsupported_and_invalid(gpu_lib):
    dev = torch.device("cuda")
    def mk(Dk, Dv, Hk=1, Hv=1):
        q = torch.zeros(1, 4, Hk, Dk, dtype=torch.bfloat16, device=dev)
        v = torch.zeros(1, 4, Hv, Dv, dtype=torch.bfloat16, device=dev)
        g = torch.zeros(1, 4, Hv, device=dev)
        return q, q.clone(), v, g, g.clone()
    for Dk, Dv, status in ((264, 64, 4), (64, 12, 4), (12, 64, 4)):
        with pytest.raises(gpu_lib.RglruError) as e:
            gpu_lib.rglru_delta_rule_fwd(*mk(Dk, Dv))
        assert e.value.status == status
    with pytest.raises(gpu_lib.RglruError) as e:
        gpu_lib.rglru_delta_rule_fwd(*mk(64, 64, Hk=2, Hv=3))
    assert e.value.status == 1
