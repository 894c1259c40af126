"""Pins of the float64 gated delta rule oracle (GDN and KDA) against facts fixed outside it.

A hand-worked two-token example (tests/golden/delta_hand.json), closed forms
(no write: pure decay of the initial state; unit writes along orthonormal
keys: exact recall of every stored value), the read-back identity of one
write, the chunk-form algebra against the token recurrence, and the layout
identities (packed sequences, grouped key heads, the value-first state). A
dropped decay, a sign slip in the error term, a transposed state or a key
head taken from the wrong group fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import chunk_gdn, recurrent_delta_rule

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _expr(e):
    return eval(e, {"__builtins__": {}}, {"log": math.log})


def _golden():
    with open(os.path.join(GOLDEN, "delta_hand.json")) as f:
        return json.load(f)


def _golden_inputs(gd, kda):
    inp = gd["inputs"]
    q = np.array(inp["q"]).reshape(1, 2, 1, 2)
    k = np.array(inp["k"]).reshape(1, 2, 1, 2)
    v = np.array(inp["v"]).reshape(1, 2, 1, 2)
    beta = np.array(inp["beta"]).reshape(1, 2, 1)
    if kda:
        g = np.array([[_expr(e) for e in row] for row in inp["g_kda_expr"]]).reshape(1, 2, 1, 2)
    else:
        g = np.array([_expr(e) for e in inp["g_gdn_expr"]]).reshape(1, 2, 1)
    h0 = np.array(inp["S0"]).reshape(1, 1, 2, 2)
    return q, k, v, g, beta, h0, inp["scale"]


def _rand(rng, B, T, Hk, Hv, Dk, Dv, kda=False, unit_keys=True):
    q = rng.standard_normal((B, T, Hk, Dk))
    k = rng.standard_normal((B, T, Hk, Dk))
    if unit_keys:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, Hv, Dv))
    g = -rng.uniform(0.01, 0.6, (B, T, Hv, Dk) if kda else (B, T, Hv))
    beta = rng.uniform(0.05, 1.0, (B, T, Hv))
    return q, k, v, g, beta


@pytest.mark.parametrize("kda", [False, True])
def test_hand_worked_two_tokens(kda):
    gd = _golden()
    q, k, v, g, beta, h0, scale = _golden_inputs(gd, kda)
    o, s = recurrent_delta_rule(q, k, v, g, beta, scale=scale, initial_state=h0)
    want = gd["kda" if kda else "gdn"]
    np.testing.assert_allclose(o[0, :, 0], want["o"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(s[0, 0], want["S_final"], rtol=0, atol=1e-14)


def test_hand_worked_chunk_form():
    gd = _golden()
    q, k, v, g, beta, h0, scale = _golden_inputs(gd, False)
    for C in (1, 2, 64):
        o, s = chunk_gdn(q, k, v, g, beta, chunk_size=C, scale=scale, initial_state=h0)
        np.testing.assert_allclose(o[0, :, 0], gd["gdn"]["o"], rtol=0, atol=1e-14)
        np.testing.assert_allclose(s[0, 0], gd["gdn"]["S_final"], rtol=0, atol=1e-14)


def test_default_scale_is_inverse_sqrt_dk():
    gd = _golden()
    q, k, v, g, beta, h0, _ = _golden_inputs(gd, False)
    o, _ = recurrent_delta_rule(q, k, v, g, beta, initial_state=h0)
    np.testing.assert_allclose(o[0, :, 0], np.array(gd["gdn"]["o"]) / math.sqrt(2.0), rtol=1e-15)


@pytest.mark.parametrize("kda", [False, True])
def test_no_write_is_pure_decay(kda):
    """beta = 0: the state only decays; o_t = scale (D_0..t S0)^T q_t with the cumulative decay."""
    rng = np.random.default_rng(1)
    B, T, H, Dk, Dv = 2, 23, 2, 5, 3
    q, k, v, g, beta = _rand(rng, B, T, H, H, Dk, Dv, kda)
    beta[:] = 0.0
    h0 = rng.standard_normal((B, H, Dk, Dv))
    o, s = recurrent_delta_rule(q, k, v, g, beta, scale=0.7, initial_state=h0)
    G = np.cumsum(g, axis=1)                              # [B, T, H] or [B, T, H, Dk]
    for b in range(B):
        for h in range(H):
            for t in range(T):
                dec = np.exp(G[b, t, h])
                St = (dec[:, None] if kda else dec) * h0[b, h]
                np.testing.assert_allclose(o[b, t, h], 0.7 * St.T @ q[b, t, h], rtol=1e-12, atol=1e-14)
            dec = np.exp(G[b, -1, h])
            np.testing.assert_allclose(s[b, h], (dec[:, None] if kda else dec) * h0[b, h], rtol=1e-12)


def test_orthonormal_unit_writes_recall_exactly():
    """No decay, beta = 1, keys orthonormal, S0 = 0: S = sum_j k_j v_j^T, so every read-out is
    o_t = scale sum_{j<=t} (q_t . k_j) v_j and S^T k_j = v_j for every stored key."""
    rng = np.random.default_rng(2)
    T, Dk, Dv = 6, 8, 4
    Qm, _ = np.linalg.qr(rng.standard_normal((Dk, Dk)))
    k = Qm[:T].reshape(1, T, 1, Dk)
    q = rng.standard_normal((1, T, 1, Dk))
    v = rng.standard_normal((1, T, 1, Dv))
    g = np.zeros((1, T, 1))
    beta = np.ones((1, T, 1))
    o, s = recurrent_delta_rule(q, k, v, g, beta, scale=1.0)
    for t in range(T):
        want = sum((q[0, t, 0] @ k[0, j, 0]) * v[0, j, 0] for j in range(t + 1))
        np.testing.assert_allclose(o[0, t, 0], want, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(s[0, 0].T @ k[0, :, 0].T, v[0, :, 0].T, atol=1e-13)


def test_repeated_key_overwrites():
    """beta = 1 along the same unit key twice: the second value replaces the first."""
    k = np.array([0.0, 0.6, 0.8]).reshape(1, 1, 1, 3).repeat(2, axis=1)
    v = np.array([[5.0, -1.0], [2.0, 7.0]]).reshape(1, 2, 1, 2)
    q = k.copy()
    o, s = recurrent_delta_rule(q, k, v, np.zeros((1, 2, 1)), np.ones((1, 2, 1)), scale=1.0)
    np.testing.assert_allclose(o[0, :, 0], v[0, :, 0], atol=1e-14)
    np.testing.assert_allclose(s[0, 0], np.outer(k[0, 0, 0], v[0, 1, 0]), atol=1e-14)


@pytest.mark.parametrize("kda", [False, True])
def test_one_write_read_back_identity(kda):
    """One token, unit key, any beta and S0: the final state read with k is
    (1 - beta) (D S0)^T k + beta v, and along directions orthogonal to k the state is D S0."""
    rng = np.random.default_rng(3)
    Dk, Dv = 7, 5
    q, k, v, g, beta = _rand(rng, 1, 1, 1, 1, Dk, Dv, kda)
    h0 = rng.standard_normal((1, 1, Dk, Dv))
    _, s = recurrent_delta_rule(q, k, v, g, beta, initial_state=h0)
    kk, b = k[0, 0, 0], beta[0, 0, 0]
    dec = np.exp(g[0, 0, 0])
    Sd = (dec[:, None] if kda else dec) * h0[0, 0]
    np.testing.assert_allclose(s[0, 0].T @ kk, (1 - b) * Sd.T @ kk + b * v[0, 0, 0], rtol=1e-12, atol=1e-13)
    P = np.eye(Dk) - np.outer(kk, kk)
    np.testing.assert_allclose(P @ s[0, 0], P @ Sd, atol=1e-13)


def test_kda_with_uniform_rows_is_gdn():
    rng = np.random.default_rng(4)
    q, k, v, g, beta = _rand(rng, 2, 19, 1, 2, 6, 4)
    h0 = rng.standard_normal((2, 2, 6, 4))
    o1, s1 = recurrent_delta_rule(q, k, v, g, beta, initial_state=h0)
    o2, s2 = recurrent_delta_rule(q, k, v, np.repeat(g[..., None], 6, axis=-1), beta, initial_state=h0)
    np.testing.assert_allclose(o1, o2, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(s1, s2, rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("C", [1, 4, 16, 64])
def test_chunk_form_equals_token_recurrence(C):
    """The chunk algebra (one unit-lower-triangular solve per chunk) is exact; both forms
    agree to rounding at every chunk size, ragged tails included."""
    rng = np.random.default_rng(5)
    q, k, v, g, beta = _rand(rng, 2, 45, 2, 4, 8, 6)
    h0 = rng.standard_normal((2, 4, 8, 6))
    o1, s1 = recurrent_delta_rule(q, k, v, g, beta, initial_state=h0)
    o2, s2 = chunk_gdn(q, k, v, g, beta, chunk_size=C, initial_state=h0)
    np.testing.assert_allclose(o2, o1, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(s2, s1, rtol=1e-11, atol=1e-12)


def test_packed_sequences_equal_separate_calls():
    rng = np.random.default_rng(7)
    lens = [5, 0, 17, 1, 9]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = int(cu[-1])
    for kda in (False, True):
        q, k, v, g, beta = _rand(rng, 1, T, 2, 2, 6, 5, kda)
        h0 = rng.standard_normal((len(lens), 2, 6, 5))
        o, s = recurrent_delta_rule(q, k, v, g, beta, initial_state=h0, cu_seqlens=cu)
        for n in range(len(lens)):
            a, b = cu[n], cu[n + 1]
            on, sn = recurrent_delta_rule(q[:, a:b], k[:, a:b], v[:, a:b], g[:, a:b], beta[:, a:b],
                                          initial_state=h0[n:n + 1])
            np.testing.assert_array_equal(o[:, a:b], on)
            np.testing.assert_array_equal(s[n], sn[0])
        if not kda:
            oc, sc = chunk_gdn(q, k, v, g, beta, chunk_size=4, initial_state=h0, cu_seqlens=cu)
            np.testing.assert_allclose(oc, o, rtol=1e-11, atol=1e-12)
            np.testing.assert_allclose(sc, s, rtol=1e-11, atol=1e-12)


def test_empty_sequence_returns_initial_state():
    rng = np.random.default_rng(8)
    q, k, v, g, beta = _rand(rng, 1, 0, 1, 1, 4, 3)
    h0 = rng.standard_normal((1, 1, 4, 3))
    o, s = recurrent_delta_rule(q, k, v, g, beta, initial_state=h0)
    assert o.shape == (1, 0, 1, 3)
    np.testing.assert_array_equal(s, h0)


def test_grouped_key_heads_equal_repeated_heads():
    """Hv = 3 Hk: value head h reads key head h // 3, the same as repeating each key head 3 times."""
    rng = np.random.default_rng(9)
    q, k, v, g, beta = _rand(rng, 2, 11, 2, 6, 4, 3, kda=True)
    o1, s1 = recurrent_delta_rule(q, k, v, g, beta)
    o2, s2 = recurrent_delta_rule(np.repeat(q, 3, axis=2), np.repeat(k, 3, axis=2), v, g, beta)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(s1, s2)


def test_value_first_state_is_the_transpose():
    rng = np.random.default_rng(10)
    q, k, v, g, beta = _rand(rng, 2, 9, 1, 1, 5, 3)
    h0 = rng.standard_normal((2, 1, 5, 3))
    o1, s1 = recurrent_delta_rule(q, k, v, g, beta, initial_state=h0)
    o2, s2 = recurrent_delta_rule(q, k, v, g, beta, initial_state=h0.transpose(0, 1, 3, 2),
                                  state_v_first=True)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(s1.transpose(0, 1, 3, 2), s2)


def test_rejects_bad_layouts():
    rng = np.random.default_rng(11)
    q, k, v, g, beta = _rand(rng, 2, 4, 2, 3, 4, 3)
    with pytest.raises(ValueError):
        recurrent_delta_rule(q, k, v, g, beta)                       # 3 % 2 != 0
    q, k, v, g, beta = _rand(rng, 2, 4, 1, 1, 4, 3)
    with pytest.raises(ValueError):
        recurrent_delta_rule(q, k, v, g, beta, cu_seqlens=[0, 4])    # packed needs B = 1
    with pytest.raises(ValueError):
        chunk_gdn(q, k, v, np.zeros((2, 4, 1, 4)), beta)             # chunk form is GDN only


# --------------------------------------------------------------- backward

from oracle import recurrent_delta_rule_backward  # noqa: E402


def _loss_fd(args, do, dhl, kw, i, idx, eps=1e-6):
    def L(a):
        o, s = recurrent_delta_rule(*a, **kw)
        return np.sum(o * do) + (np.sum(s * dhl) if dhl is not None else 0.0)
    ap = [x.copy() for x in args]
    am = [x.copy() for x in args]
    ap[i][idx] += eps
    am[i][idx] -= eps
    return (L(ap) - L(am)) / (2 * eps)


@pytest.mark.parametrize("kda", [False, True])
@pytest.mark.parametrize("layout", ["rows", "packed", "v_first"])
def test_backward_matches_finite_differences(kda, layout):
    """Every gradient, element by element, against central differences of <do, o> + <dh_last, S_final>."""
    rng = np.random.default_rng(20 + kda)
    B, T, Hk, Hv, Dk, Dv = (2, 5, 1, 2, 3, 2) if layout != "packed" else (1, 7, 1, 2, 3, 2)
    q, k, v, g, beta = _rand(rng, B, T, Hk, Hv, Dk, Dv, kda)
    cu = [0, 3, 3, 7] if layout == "packed" else None
    N = 3 if layout == "packed" else B
    vf = layout == "v_first"
    sshape = (N, Hv, Dv, Dk) if vf else (N, Hv, Dk, Dv)
    h0 = rng.standard_normal(sshape)
    do = rng.standard_normal((B, T, Hv, Dv))
    dhl = rng.standard_normal(sshape)
    kw = dict(scale=0.7, initial_state=h0, cu_seqlens=cu, state_v_first=vf)
    grads = recurrent_delta_rule_backward(q, k, v, g, beta, do, dhl, **kw)
    args = [q, k, v, g, beta]
    for i, gr in enumerate(grads[:5]):
        fd = np.zeros_like(args[i])
        for idx in np.ndindex(*args[i].shape):
            fd[idx] = _loss_fd(args, do, dhl, kw, i, idx)
        np.testing.assert_allclose(gr, fd, rtol=1e-6, atol=1e-7, err_msg=f"input {i}")
    # initial state
    def L0(h):
        o, s = recurrent_delta_rule(q, k, v, g, beta, **dict(kw, initial_state=h))
        return np.sum(o * do) + np.sum(s * dhl)
    fd = np.zeros_like(h0)
    for idx in np.ndindex(*h0.shape):
        hp, hm = h0.copy(), h0.copy()
        hp[idx] += 1e-6
        hm[idx] -= 1e-6
        fd[idx] = (L0(hp) - L0(hm)) / 2e-6
    np.testing.assert_allclose(grads[5], fd, rtol=1e-6, atol=1e-7)


def test_backward_without_writes_is_closed_form():
    """beta = 0: S_t = Gamma_t S0, so dh0 = sum_t scale Gamma_t q_t do_t^T + Gamma_T dh_last, dv = 0."""
    rng = np.random.default_rng(30)
    T, Dk, Dv = 9, 4, 3
    q, k, v, g, beta = _rand(rng, 1, T, 1, 1, Dk, Dv)
    beta[:] = 0.0
    do = rng.standard_normal((1, T, 1, Dv))
    dhl = rng.standard_normal((1, 1, Dk, Dv))
    dq, dk, dv, dg, db, dh0 = recurrent_delta_rule_backward(q, k, v, g, beta, do, dhl, scale=0.5)
    Gam = np.exp(np.cumsum(g[0, :, 0]))
    want = sum(0.5 * Gam[t] * np.outer(q[0, t, 0], do[0, t, 0]) for t in range(T)) + Gam[-1] * dhl[0, 0]
    np.testing.assert_allclose(dh0[0, 0], want, rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(dv, 0.0)
    np.testing.assert_array_equal(dq, 0.0)   # zero state and no writes: o = 0 for any q


@pytest.mark.parametrize("kda", [False, True])
def test_backward_of_one_write_from_zero_is_closed_form(kda):
    """One token from a zero state: S = beta k v^T and o = scale beta (k.q) v, so with
    L = dh_last and G = scale q do^T + L (derived by hand):
      dq = scale beta (v.do) k,  dk = scale beta (v.do) q + beta L v,
      dv = scale beta (k.q) do + beta L^T k,  dbeta = scale (k.q)(v.do) + k^T L v,
      dg = 0 (the decay only scales the zero state),  dh0 = D (I - beta k k^T) G."""
    rng = np.random.default_rng(32)
    Dk, Dv, sc = 4, 3, 0.7
    q, k, v, g, beta = _rand(rng, 1, 1, 1, 1, Dk, Dv, kda=kda)
    do = rng.standard_normal((1, 1, 1, Dv))
    L = rng.standard_normal((1, 1, Dk, Dv))
    dq, dk, dv, dg, db, dh0 = recurrent_delta_rule_backward(q, k, v, g, beta, do, L, scale=sc)
    qv, kv, vv, dov, Lm, b = q[0, 0, 0], k[0, 0, 0], v[0, 0, 0], do[0, 0, 0], L[0, 0], beta[0, 0, 0]
    kq, vdo = kv @ qv, vv @ dov
    np.testing.assert_allclose(dq[0, 0, 0], sc * b * vdo * kv, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dk[0, 0, 0], sc * b * vdo * qv + b * (Lm @ vv), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dv[0, 0, 0], sc * b * kq * dov + b * (Lm.T @ kv), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(db[0, 0, 0], sc * kq * vdo + kv @ Lm @ vv, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dg, 0.0, atol=1e-15)
    D = np.diag(np.exp(g[0, 0, 0])) if kda else np.exp(g[0, 0, 0]) * np.eye(Dk)
    G = sc * np.outer(qv, dov) + Lm
    np.testing.assert_allclose(dh0[0, 0], D @ (np.eye(Dk) - b * np.outer(kv, kv)) @ G, rtol=1e-12, atol=1e-14)


def test_backward_is_linear_in_the_output_gradients():
    rng = np.random.default_rng(31)
    q, k, v, g, beta = _rand(rng, 1, 6, 1, 2, 4, 3, kda=True)
    h0 = rng.standard_normal((1, 2, 4, 3))
    d1, d2 = rng.standard_normal((2, 1, 6, 2, 3))
    l1, l2 = rng.standard_normal((2, 1, 2, 4, 3))
    a = recurrent_delta_rule_backward(q, k, v, g, beta, d1, l1, initial_state=h0)
    b = recurrent_delta_rule_backward(q, k, v, g, beta, d2, l2, initial_state=h0)
    c = recurrent_delta_rule_backward(q, k, v, g, beta, 2 * d1 - d2, 2 * l1 - l2, initial_state=h0)
    for x, y, z in zip(a, b, c):
        np.testing.assert_allclose(z, 2 * x - y, rtol=1e-10, atol=1e-12)
