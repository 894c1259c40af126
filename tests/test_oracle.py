"""Pins of the float64 oracle against facts fixed outside it.

Closed forms, exact limits, a hand-built reset sequence (tests/golden), the
stationarity identity of the normalized write, linearity, the exact chunked
composition, and central finite differences. Each is chosen so a plausible
slip in the oracle (a dropped term, a wrong sign, an index off by one, the
wrong constant, a transposed block) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
SQ3 = math.sqrt(3.0)


def _expr(e):
    return eval(e, {"__builtins__": {}}, {"sqrt": math.sqrt, "log": math.log, "expm1": math.expm1})


# --------------------------------------------------------------- primitives

def test_sigmoid_softplus_reference_values():
    assert oracle.sigmoid(np.array([0.0]))[0] == 0.5
    np.testing.assert_allclose(oracle.sigmoid(np.array([2.0, -2.0])),
                               [1 / (1 + math.exp(-2)), math.exp(-2) / (1 + math.exp(-2))], rtol=1e-15)
    assert oracle.sigmoid(np.array([-800.0]))[0] == 0.0
    assert oracle.sigmoid(np.array([800.0]))[0] == 1.0
    np.testing.assert_allclose(oracle.softplus(np.array([0.0, 30.0, -30.0])),
                               [math.log(2.0), 30.0 + math.log1p(math.exp(-30)), math.log1p(math.exp(-30))],
                               rtol=1e-15)


def test_multiplier_is_sqrt_one_minus_a_squared():
    rng = np.random.default_rng(0)
    gx = rng.standard_normal((1, 50, 4))
    ga = rng.standard_normal((1, 50, 4))
    lam = rng.uniform(-9, 3, 4)
    i, r, s, l, a, m = oracle.gates(gx, ga, lam)
    np.testing.assert_allclose(m, np.sqrt(1 - a * a), rtol=1e-9)
    np.testing.assert_allclose(a, np.exp(-8.0 * np.log1p(np.exp(lam)) * r), rtol=1e-14)


# --------------------------------------------------------------- forward pins

def test_constant_gates_geometric_series():
    """Constant gates and input: h_t = a^(t+1) h0 + m i X (1 - a^(t+1)) / (1 - a)."""
    B, L, W = 2, 40, 3
    gxv = np.array([0.3, -1.2, 2.0])
    gav = np.array([-0.7, 0.5, 1.5])
    X = np.array([[1.5, -0.25, 3.0], [-2.0, 0.75, 0.5]])
    lam = np.array([-4.0, -2.5, -6.0])
    h0 = np.array([[0.5, -1.0, 2.0], [1.0, 0.0, -3.0]])
    x = np.broadcast_to(X[:, None, :], (B, L, W)).copy()
    gx = np.broadcast_to(gxv, (B, L, W)).copy()
    ga = np.broadcast_to(gav, (B, L, W)).copy()
    h, h_last = oracle.rglru_forward(x, gx, ga, lam, None, h0)
    i = 1 / (1 + np.exp(-gxv))
    r = 1 / (1 + np.exp(-gav))
    a = np.exp(-8 * np.log1p(np.exp(lam)) * r)
    m = np.sqrt(1 - a ** 2)
    t = np.arange(L)[None, :, None]
    expect = a ** (t + 1) * h0[:, None, :] + m * i * X[:, None, :] * (1 - a ** (t + 1)) / (1 - a)
    np.testing.assert_allclose(h, expect, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(h_last, expect[:, -1], rtol=1e-10, atol=1e-12)


def test_fast_decay_limit_gives_gated_input_exactly():
    """A huge lam makes a underflow to 0, so m = 1 and h = i * x exactly."""
    rng = np.random.default_rng(1)
    x, gx, ga = (rng.standard_normal((2, 9, 5)) for _ in range(3))
    lam = np.full(5, 1e6)
    h, _ = oracle.rglru_forward(x, gx, ga, lam, None, rng.standard_normal((2, 5)))
    np.testing.assert_array_equal(h, oracle.sigmoid(gx) * x)


def test_no_decay_limit_keeps_initial_state_exactly():
    """lam = -800 makes softplus 0, so a = 1, m = 0 and the state never moves."""
    rng = np.random.default_rng(2)
    x, gx, ga = (rng.standard_normal((2, 9, 5)) for _ in range(3))
    h0 = rng.standard_normal((2, 5))
    h, _ = oracle.rglru_forward(x, gx, ga, np.full(5, -800.0), None, h0)
    np.testing.assert_array_equal(h, np.broadcast_to(h0[:, None, :], h.shape))


def _golden():
    with open(os.path.join(GOLDEN, "reset_hand.json")) as f:
        return json.load(f)


def _golden_inputs(g):
    inp = g["inputs"]
    L = len(inp["x"])
    x = np.array(inp["x"]).reshape(1, L, 1)
    gx = np.full((1, L, 1), inp["gate_x"])
    ga = np.full((1, L, 1), inp["gate_a"])
    lam = np.array([_expr(inp["lam_expr"])])
    reset = np.array(inp["reset"], dtype=np.uint8).reshape(1, L)
    h0 = np.array([[inp["h0"]]])
    dh = np.array(inp["dh"]).reshape(1, L, 1)
    return x, gx, ga, lam, reset, h0, dh


def test_golden_fixture_is_self_consistent():
    g = _golden()
    for e, v in zip(g["forward"]["h_expr"], g["forward"]["h"]):
        assert abs(_expr(e) - v) < 1e-15 * max(1.0, abs(v))
    for e, v in zip(g["backward"]["dx_expr"], g["backward"]["dx"]):
        assert abs(_expr(e) - v) < 1e-15 * max(1.0, abs(v))
    assert abs(_expr(g["backward"]["dlam_expr"]) - g["backward"]["dlam"]) < 1e-14


def test_hand_built_resets_forward():
    g = _golden()
    x, gx, ga, lam, reset, h0, _ = _golden_inputs(g)
    h, h_last = oracle.rglru_forward(x, gx, ga, lam, reset, h0, c=g["inputs"]["c"])
    np.testing.assert_allclose(h[0, :, 0], g["forward"]["h"], rtol=1e-14, atol=1e-14)
    assert h[0, 0, 0] == 2.0 and h[0, 3, 0] == 8.0   # reset tokens are exact


def test_hand_built_resets_backward():
    g = _golden()
    x, gx, ga, lam, reset, h0, dh = _golden_inputs(g)
    out = oracle.rglru_backward(x, gx, ga, lam, dh, reset, h0, c=g["inputs"]["c"])
    bw = g["backward"]
    np.testing.assert_allclose(out["dx"][0, :, 0], bw["dx"], rtol=1e-14)
    np.testing.assert_array_equal(out["dgx"][0, :, 0], bw["dgx"])
    np.testing.assert_array_equal(out["dga"][0, :, 0], bw["dga"])
    np.testing.assert_allclose(out["dlam"], [bw["dlam"]], rtol=1e-13)
    assert out["dh0"][0, 0] == 0.0


def _golden_half():
    with open(os.path.join(GOLDEN, "half_gates_hand.json")) as f:
        return json.load(f)


def _half_inputs(g):
    inp = g["inputs"]
    L = len(inp["x"])
    x = np.array(inp["x"]).reshape(1, L, 1)
    gx = np.full((1, L, 1), inp["gate_x"])
    ga = np.full((1, L, 1), inp["gate_a"])
    lam = np.array([_expr(inp["lam_expr"])])
    h0 = np.array([[inp["h0"]]])
    dh = np.array(inp["dh"]).reshape(1, L, 1)
    dh_last = np.array([[inp["dh_last"]]])
    return x, gx, ga, lam, h0, dh, dh_last


def test_half_gates_fixture_is_self_consistent():
    g = _golden_half()
    for e, v in zip(g["forward"]["h_expr"], g["forward"]["h"]):
        assert abs(_expr(e) - v) <= 1e-15 * max(1.0, abs(v))
    bw = g["backward"]
    for k in ("dx", "dgx", "dga"):
        for e, v in zip(bw[k + "_expr"], bw[k]):
            assert abs(_expr(e) - v) <= 1e-15 * max(1.0, abs(v)), k
    assert abs(_expr(bw["dlam_expr"]) - bw["dlam"]) <= 1e-15
    assert _expr(bw["dh0_expr"]) == bw["dh0"]


def test_half_gates_forward():
    # gates at 0: the sigmoids give exactly 1/2 and a is exactly 1/2
    g = _golden_half()
    x, gx, ga, lam, h0, _, _ = _half_inputs(g)
    h, h_last = oracle.rglru_forward(x, gx, ga, lam, None, h0, c=g["inputs"]["c"])
    expect = [_expr(e) for e in g["forward"]["h_expr"]]
    np.testing.assert_allclose(h[0, :, 0], expect, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(h_last[0], [_expr(g["forward"]["h_last_expr"])], rtol=1e-14)


def test_half_gates_backward():
    # every gradient of the hand derivation, nonzero gate derivatives included
    g = _golden_half()
    x, gx, ga, lam, h0, dh, dh_last = _half_inputs(g)
    out = oracle.rglru_backward(x, gx, ga, lam, dh, None, h0, dh_last, c=g["inputs"]["c"])
    bw = g["backward"]
    for k in ("dx", "dgx", "dga"):
        expect = [_expr(e) for e in bw[k + "_expr"]]
        np.testing.assert_allclose(out[k][0, :, 0], expect, rtol=1e-14, atol=1e-14, err_msg=k)
    np.testing.assert_allclose(out["dlam"], [_expr(bw["dlam_expr"])], rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(out["dh0"][0], [_expr(bw["dh0_expr"])], rtol=1e-14, atol=1e-14)


def _golden_varlen():
    with open(os.path.join(GOLDEN, "varlen_hand.json")) as f:
        return json.load(f)


def test_varlen_hand_built():
    # three packed sequences, one of them empty, a reset token in the last:
    # every state, final state and gradient of the hand derivation
    g = _golden_varlen()
    inp = g["inputs"]
    T, n = len(inp["x"]), len(inp["cu_seqlens"]) - 1
    x = np.array(inp["x"]).reshape(T, 1)
    gx = np.full((T, 1), inp["gate_x"])
    ga = np.full((T, 1), inp["gate_a"])
    lam = np.array([_expr(inp["lam_expr"])])
    reset = np.array(inp["reset"], dtype=np.uint8)
    h0 = np.array(inp["h0"]).reshape(n, 1)
    dh = np.array(inp["dh"]).reshape(T, 1)
    dh_last = np.array(inp["dh_last"]).reshape(n, 1)
    h, h_last = oracle.rglru_forward_varlen(x, gx, ga, lam, inp["cu_seqlens"], reset, h0, c=inp["c"])
    np.testing.assert_allclose(h[:, 0], [_expr(e) for e in g["forward"]["h_expr"]], rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(h_last[:, 0], [_expr(e) for e in g["forward"]["h_last_expr"]], rtol=1e-14)
    out = oracle.rglru_backward_varlen(x, gx, ga, lam, dh, inp["cu_seqlens"], reset, h0, dh_last, c=inp["c"])
    for k in ("dx", "dgx"):
        np.testing.assert_allclose(out[k][:, 0], [_expr(e) for e in g["backward"][k + "_expr"]], rtol=1e-14,
                                   atol=1e-14, err_msg=k)
    np.testing.assert_allclose(out["dh0"][:, 0], [_expr(e) for e in g["backward"]["dh0_expr"]], rtol=1e-14)
    assert out["dga"][3, 0] == 0.0   # reset token


def test_varlen_with_a_reset_at_every_start_is_one_row():
    # Zero initial states and a reset token on every sequence's first token:
    # no state crosses a boundary either way, so the packed sequences are the
    # one-row recurrence with those resets (an independent route through the
    # row oracle's reset handling).
    rng = np.random.default_rng(11)
    lens = [5, 1, 0, 9, 3, 0, 12]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T, W = int(cu[-1]), 4
    x, gx, ga, dh = (rng.standard_normal((T, W)) for _ in range(4))
    lam = rng.uniform(-6, 1, W)
    user = (rng.random(T) < 0.15).astype(np.uint8)
    starts = np.zeros(T, dtype=np.uint8)
    starts[cu[:-1][np.array(lens) > 0]] = 1
    reset = np.maximum(user, starts)
    h, h_last = oracle.rglru_forward_varlen(x, gx, ga, lam, cu, reset)
    hr, _ = oracle.rglru_forward(x[None], gx[None], ga[None], lam, reset[None])
    np.testing.assert_array_equal(h, hr[0])
    for k, (lo, hi) in enumerate(zip(cu[:-1], cu[1:])):
        np.testing.assert_array_equal(h_last[k], hr[0, hi - 1] if hi > lo else 0.0)
    out = oracle.rglru_backward_varlen(x, gx, ga, lam, dh, cu, reset)
    ref = oracle.rglru_backward(x[None], gx[None], ga[None], lam, dh[None], reset[None])
    for k in ("dx", "dgx", "dga"):
        np.testing.assert_array_equal(out[k], ref[k][0])
    np.testing.assert_allclose(out["dlam"], ref["dlam"], rtol=1e-13)
    np.testing.assert_array_equal(out["dh0"], 0.0)


# --------------------------------------------------------------- stationarity

@pytest.mark.parametrize("with_h0", [False, True])
def test_stationarity_identity(with_h0):
    """With i = 1 the normalized write keeps unit gain: for every t,
    sum_s (dh_t/dx_s)^2 + (dh_t/dh0)^2 = 1, where a reset at t = 0 removes the
    h0 term. The sensitivities come from the oracle backward with dh = e_t, so
    this also ties the backward to the forward."""
    rng = np.random.default_rng(3)
    B, L, W = 1, 30, 4
    x = rng.standard_normal((B, L, W))
    gx = np.full((B, L, W), 40.0)                 # i == 1.0 exactly
    ga = rng.standard_normal((B, L, W)) * 2
    lam = rng.uniform(-6, 1, W)
    reset = np.zeros((B, L), dtype=np.uint8)
    reset[0, 12] = 1                              # a reset mid-way keeps the identity
    h0 = rng.standard_normal((B, W)) if with_h0 else None
    if not with_h0:
        reset[0, 0] = 1
    for t in [0, 1, 5, 11, 12, 13, 29]:
        dh = np.zeros((B, L, W))
        dh[:, t, :] = 1.0
        g = oracle.rglru_backward(x, gx, ga, lam, dh, reset, h0)
        total = np.sum(g["dx"] ** 2, axis=1)
        if with_h0:
            total = total + g["dh0"] ** 2
        np.testing.assert_allclose(total, 1.0, rtol=1e-12)


def test_stationary_variance_monte_carlo():
    """iid unit-variance inputs and initial state, constant gates, i = 1: Var(h_t) stays 1."""
    rng = np.random.default_rng(4)
    B, L, W = 4096, 64, 2
    x = rng.standard_normal((B, L, W))
    gx = np.full((B, L, W), 40.0)
    ga = np.broadcast_to(np.array([0.3, -1.0]), (B, L, W)).copy()
    lam = np.array([-3.0, -5.0])
    h0 = rng.standard_normal((B, W))
    h, _ = oracle.rglru_forward(x, gx, ga, lam, None, h0)
    var = h.var(axis=0)
    # the sample variance of B normals has std sqrt(2/B)
    assert np.all(np.abs(var - 1.0) < 5 * math.sqrt(2.0 / B))


def test_linear_in_input_and_initial_state():
    rng = np.random.default_rng(5)
    B, L, W = 2, 17, 3
    gx, ga = rng.standard_normal((B, L, W)), rng.standard_normal((B, L, W))
    lam = rng.uniform(-8, 0, W)
    reset = (rng.random((B, L)) < 0.2).astype(np.uint8)
    x1, x2 = rng.standard_normal((B, L, W)), rng.standard_normal((B, L, W))
    p1, p2 = rng.standard_normal((B, W)), rng.standard_normal((B, W))
    h1, _ = oracle.rglru_forward(x1, gx, ga, lam, reset, p1)
    h2, _ = oracle.rglru_forward(x2, gx, ga, lam, reset, p2)
    h3, _ = oracle.rglru_forward(2 * x1 - 3 * x2, gx, ga, lam, reset, 2 * p1 - 3 * p2)
    np.testing.assert_allclose(h3, 2 * h1 - 3 * h2, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------- chunked composition

@pytest.mark.parametrize("chunk", [1, 3, 7, 16, 36, 37, 42])
def test_chunked_equals_sequential(chunk):
    rng = np.random.default_rng(6)
    B, L, W = 3, 37, 4
    x, gx, ga = (rng.standard_normal((B, L, W)) for _ in range(3))
    lam = rng.uniform(-9, -1, W)
    reset = (rng.random((B, L)) < 0.1).astype(np.uint8)
    h0 = rng.standard_normal((B, W))
    h, hl = oracle.rglru_forward(x, gx, ga, lam, reset, h0)
    hc, hlc = oracle.rglru_forward_chunked(x, gx, ga, lam, reset, h0, chunk=chunk)
    np.testing.assert_allclose(hc, h, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(hlc, hl, rtol=1e-13, atol=1e-13)


# --------------------------------------------------------------- backward

def _loss(x, gx, ga, lam, reset, h0, dh, dh_last):
    h, hl = oracle.rglru_forward(x, gx, ga, lam, reset, h0)
    return float(np.sum(dh * h) + np.sum(dh_last * hl))


def test_backward_matches_central_differences():
    rng = np.random.default_rng(7)
    B, L, W = 2, 7, 3
    x, gx, ga = (rng.standard_normal((B, L, W)) for _ in range(3))
    lam = rng.uniform(-5, 0.5, W)
    reset = np.zeros((B, L), dtype=np.uint8)
    reset[0, 3] = 1
    reset[1, 5] = 1
    h0 = rng.standard_normal((B, W))
    dh = rng.standard_normal((B, L, W))
    dh_last = rng.standard_normal((B, W))
    g = oracle.rglru_backward(x, gx, ga, lam, dh, reset, h0, dh_last)
    eps = 1e-6
    args = {"x": x, "gx": gx, "ga": ga, "lam": lam, "h0": h0}
    names = {"x": "dx", "gx": "dgx", "ga": "dga", "lam": "dlam", "h0": "dh0"}
    for name, arr in args.items():
        fd = np.empty_like(arr)
        for idx in np.ndindex(arr.shape):
            p = {k: v.copy() for k, v in args.items()}
            p[name][idx] += eps
            lp = _loss(p["x"], p["gx"], p["ga"], p["lam"], reset, p["h0"], dh, dh_last)
            p[name][idx] -= 2 * eps
            lm = _loss(p["x"], p["gx"], p["ga"], p["lam"], reset, p["h0"], dh, dh_last)
            fd[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(g[names[name]], fd, rtol=1e-6, atol=1e-7, err_msg=name)


def test_backward_exact_zeros_at_resets():
    rng = np.random.default_rng(8)
    B, L, W = 2, 20, 4
    x, gx, ga, dh = (rng.standard_normal((B, L, W)) for _ in range(4))
    lam = rng.uniform(-8, -2, W)
    reset = np.zeros((B, L), dtype=np.uint8)
    reset[:, 0] = 1
    reset[0, 9] = 1
    reset[1, 14] = 1
    h0 = rng.standard_normal((B, W))
    g = oracle.rglru_backward(x, gx, ga, lam, dh, reset, h0)
    assert np.all(g["dga"][reset.astype(bool)] == 0.0)
    np.testing.assert_array_equal(g["dh0"], 0.0)
    # gradients before a reset do not depend on dh after it
    dh2 = dh.copy()
    dh2[0, 9:] = rng.standard_normal((L - 9, W))
    g2 = oracle.rglru_backward(x, gx, ga, lam, dh2, reset, h0)
    for k in ("dx", "dgx", "dga"):
        np.testing.assert_array_equal(g2[k][0, :9], g[k][0, :9])
        np.testing.assert_array_equal(g2[k][1], g[k][1])


def test_nan_before_reset_does_not_cross():
    rng = np.random.default_rng(9)
    B, L, W = 1, 12, 3
    x, gx, ga = (rng.standard_normal((B, L, W)) for _ in range(3))
    lam = rng.uniform(-8, -2, W)
    reset = np.zeros((B, L), dtype=np.uint8)
    reset[0, 6] = 1
    h, _ = oracle.rglru_forward(x, gx, ga, lam, reset, None)
    x2 = x.copy()
    x2[0, 2, 1] = np.nan
    ga2 = ga.copy()
    ga2[0, 4, 0] = np.inf
    h2, _ = oracle.rglru_forward(x2, gx, ga2, lam, reset, None)
    np.testing.assert_array_equal(h2[:, 6:], h[:, 6:])
    assert np.isnan(h2[0, 2, 1])
    # the chunked composition isolates the reset the same way, whatever the chunking
    for chunk in (1, 4, 5, 7, 12):
        hc, _ = oracle.rglru_forward_chunked(x2, gx, ga2, lam, reset, None, chunk=chunk)
        assert np.all(np.isfinite(hc[:, 6:]))
        np.testing.assert_allclose(hc[:, 6:], h[:, 6:], rtol=1e-13, atol=1e-13)


# --------------------------------------------------------------- projection

def _dense_blockdiag(w):
    import scipy.linalg
    return scipy.linalg.block_diag(*list(w))


def test_projection_identity_zero_and_permutation():
    rng = np.random.default_rng(10)
    T, nb, bs = 5, 3, 4
    x = rng.standard_normal((T, nb * bs))
    b = rng.standard_normal(nb * bs)
    eye = np.broadcast_to(np.eye(bs), (nb, bs, bs)).copy()
    np.testing.assert_array_equal(oracle.blockdiag_proj_forward(x, eye, np.zeros(nb * bs)), x)
    np.testing.assert_array_equal(oracle.blockdiag_proj_forward(x, np.zeros((nb, bs, bs)), b),
                                  np.broadcast_to(b, (T, nb * bs)))
    # w[k] is read as [in, out]: a cyclic shift block sends input column j to output column j+1
    shift = np.zeros((nb, bs, bs))
    for k in range(nb):
        for j in range(bs):
            shift[k, j, (j + 1) % bs] = 1.0
    y = oracle.blockdiag_proj_forward(x, shift, np.zeros(nb * bs))
    for k in range(nb):
        for j in range(bs):
            np.testing.assert_array_equal(y[:, k * bs + (j + 1) % bs], x[:, k * bs + j])


def test_projection_matches_dense_block_diagonal_matrix():
    rng = np.random.default_rng(11)
    T, nb, bs = 9, 3, 5
    x = rng.standard_normal((T, nb * bs))
    w = rng.standard_normal((nb, bs, bs))
    b = rng.standard_normal(nb * bs)
    dy = rng.standard_normal((T, nb * bs))
    Wd = _dense_blockdiag(w)
    np.testing.assert_allclose(oracle.blockdiag_proj_forward(x, w, b), x @ Wd + b, rtol=1e-13, atol=1e-13)
    dx, dw, db = oracle.blockdiag_proj_backward(x, w, dy)
    np.testing.assert_allclose(dx, dy @ Wd.T, rtol=1e-13, atol=1e-13)
    dWd = x.T @ dy
    for k in range(nb):
        sl = slice(k * bs, (k + 1) * bs)
        np.testing.assert_allclose(dw[k], dWd[sl, sl], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(db, dy.sum(0), rtol=1e-13)


def test_projection_backward_central_differences():
    rng = np.random.default_rng(12)
    T, nb, bs = 3, 2, 3
    x = rng.standard_normal((T, nb * bs))
    w = rng.standard_normal((nb, bs, bs))
    b = rng.standard_normal(nb * bs)
    dy = rng.standard_normal((T, nb * bs))
    dx, dw, db = oracle.blockdiag_proj_backward(x, w, dy)

    def loss(x_, w_, b_):
        return float(np.sum(dy * oracle.blockdiag_proj_forward(x_, w_, b_)))

    eps = 1e-6
    for arr, grad, which in ((x, dx, 0), (w, dw, 1), (b, db, 2)):
        for idx in np.ndindex(arr.shape):
            p = [x.copy(), w.copy(), b.copy()]
            p[which][idx] += eps
            lp = loss(*p)
            p[which][idx] -= 2 * eps
            lm = loss(*p)
            assert abs((lp - lm) / (2 * eps) - grad[idx]) < 1e-6
