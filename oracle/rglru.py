"""Float64 CPU oracle of the fused RG-LRU (Hawk) gated linear recurrence.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import or run this module. The product path (the HIP
library and its Python binding) never calls it and shares no code with it.

What is computed, per batch row b, channel w and time t (the Fattori
comparison page lists the pieces the fused operator covers: both sigmoid
gates, softplus of a_param with a dynamic decay and the stationary
square-root factor, the input-gated write, the sequential state-stationary
recurrence, and a custom backward with the reverse recurrence and pointwise
derivatives; the constant c = 8 and the exact decay formula are the plainest
reading consistent with "softplus(a_param), dynamic decay"):

    i_t = sigmoid(gx_t)            r_t = sigmoid(ga_t)
    s   = softplus(lam_w)          l_t = -c * s * r_t          a_t = exp(l_t)
    m_t = sqrt(1 - a_t^2)          evaluated as sqrt(-expm1(2 l_t))
    reset token (canonical reset-token normalization, same page, "Semantic
    limits" list): the state is cleared and the write uses multiplier 1
    h_t = alpha_t * h_{t-1} + mult_t * i_t * x_t,  alpha_t = 0 and mult_t = 1 on
    a reset token, alpha_t = a_t and mult_t = m_t otherwise;  h_{-1} = h0 or 0.

The reset is applied as a select, so nothing from before a reset (not even a
NaN) reaches the state after it.

The backward follows the chain rule of that forward, literally and serially
in reverse time, for the loss <dh, h> + <dh_last, h_{L-1}>.

Arithmetic is float64 on the exact stored input values; nothing is rounded.
Every function here is pinned by tests/test_oracle.py against closed forms,
exact limits, a hand-built reset sequence, the stationarity identity and
finite differences.
"""
from __future__ import annotations

import numpy as np

C_DEFAULT = 8.0


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def sigmoid(z):
    """Logistic function, evaluated without overflow for either sign."""
    z = _f64(z)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = ez / (1.0 + ez)
    return out


def softplus(z):
    """log(1 + exp(z)), evaluated stably."""
    return np.logaddexp(0.0, _f64(z))


def gates(gx, ga, lam, c=C_DEFAULT):
    """Pointwise gate values of the method (input gate, recurrence gate, decay, multiplier).

    Returns i, r, s, l, a, m with s = softplus(lam) broadcast on the last axis.
    """
    i = sigmoid(gx)
    r = sigmoid(ga)
    s = softplus(lam)
    l = -c * s * r
    a = np.exp(l)
    m = np.sqrt(-np.expm1(2.0 * l))
    return i, r, s, l, a, m


def _reset_mask(reset, B, L):
    if reset is None:
        return np.zeros((B, L), dtype=bool)
    return np.asarray(reset).astype(bool).reshape(B, L)


def rglru_forward(x, gx, ga, lam, reset=None, h0=None, c=C_DEFAULT):
    """Sequential forward. Inputs [B, L, W]; lam [W]; reset [B, L] or None; h0 [B, W] or None.

    Returns (h [B, L, W], h_last [B, W]) in float64.
    """
    x = _f64(x)
    B, L, W = x.shape
    i, r, s, l, a, m = gates(gx, ga, lam, c)
    rst = _reset_mask(reset, B, L)
    h = np.empty((B, L, W))
    prev = np.zeros((B, W)) if h0 is None else _f64(h0).copy()
    for t in range(L):
        rt = rst[:, t][:, None]
        write = np.where(rt, 1.0, m[:, t]) * i[:, t] * x[:, t]
        prev = np.where(rt, write, a[:, t] * prev + write)
        h[:, t] = prev
    return h, prev.copy()


def rglru_backward(x, gx, ga, lam, dh, reset=None, h0=None, dh_last=None, c=C_DEFAULT):
    """Reverse recurrence and pointwise derivatives of rglru_forward.

    Loss convention: <dh, h> + <dh_last, h_{L-1}>. Returns a dict with
    dx, dgx, dga [B, L, W], dlam [W] (summed over batch and time) and dh0 [B, W]
    (the gradient on the initial state; zeros when the first token is a reset).
    """
    x = _f64(x)
    dh = _f64(dh)
    B, L, W = x.shape
    i, r, s, l, a, m = gates(gx, ga, lam, c)
    rst = _reset_mask(reset, B, L)
    h, _ = rglru_forward(x, gx, ga, lam, reset, h0, c)
    h_init = np.zeros((B, W)) if h0 is None else _f64(h0)

    dx = np.empty((B, L, W))
    dgx = np.empty((B, L, W))
    dga = np.empty((B, L, W))
    ds = np.zeros(W)
    # carry = d loss / d h_t arriving from step t+1 (alpha_{t+1} g_{t+1}), plus dh_last at the end
    carry = np.zeros((B, W)) if dh_last is None else _f64(dh_last).copy()
    for t in reversed(range(L)):
        rt = rst[:, t][:, None]
        g = dh[:, t] + carry
        mult = np.where(rt, 1.0, m[:, t])
        it, xt, at, rtv = i[:, t], x[:, t], a[:, t], r[:, t]
        hprev = h[:, t - 1] if t > 0 else h_init
        dx[:, t] = g * mult * it
        dgx[:, t] = g * mult * xt * it * (1.0 - it)
        # d/dl of (a * hprev + sqrt(1 - a^2) * i * x), with da/dl = a and dm/da = -a/m
        with np.errstate(divide="ignore", invalid="ignore"):
            dl_off = g * (at * hprev - at * at * it * xt / m[:, t])
        dl = np.where(rt, 0.0, dl_off)
        dga[:, t] = dl * (-c * s) * rtv * (1.0 - rtv)
        ds += np.sum(dl * (-c * rtv), axis=0)
        carry = np.where(rt, 0.0, at * g)
    dlam = ds * sigmoid(lam)
    return {"dx": dx, "dgx": dgx, "dga": dga, "dlam": dlam, "dh0": carry}


def rglru_forward_varlen(x, gx, ga, lam, cu_seqlens, reset=None, h0=None, c=C_DEFAULT):
    """Packed sequences (the cu_seqlens convention of the linear-attention
    reference oracles, recurrent_delta_rule_reference: offsets into one packed
    row, one initial and one final state per sequence).

    x, gx, ga [T, W]; cu_seqlens [n + 1] offsets, sequence s holding tokens
    cu[s] .. cu[s+1]-1; reset [T] or None; h0 [n, W] or None. Each sequence is
    its own row of rglru_forward from h0[s]. Returns (h [T, W], h_last [n, W]);
    a sequence without tokens has h_last = h0[s] (zero without h0).
    """
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    n = cu.size - 1
    T, W = np.shape(x)
    h = np.zeros((T, W))
    h_last = np.zeros((n, W)) if h0 is None else _f64(h0).copy()
    for k in range(n):
        lo, hi = int(cu[k]), int(cu[k + 1])
        if hi <= lo:
            continue
        sl = slice(lo, hi)
        hk, hl = rglru_forward(_f64(x)[None, sl], _f64(gx)[None, sl], _f64(ga)[None, sl], lam,
                               None if reset is None else np.asarray(reset)[None, sl],
                               None if h0 is None else _f64(h0)[k][None], c)
        h[sl] = hk[0]
        h_last[k] = hl[0]
    return h, h_last


def rglru_backward_varlen(x, gx, ga, lam, dh, cu_seqlens, reset=None, h0=None, dh_last=None, c=C_DEFAULT):
    """Backward of rglru_forward_varlen for the loss <dh, h> + <dh_last, h_last>.

    Returns dx, dgx, dga [T, W], dlam [W] (summed over every sequence and
    token) and dh0 [n, W]; a sequence without tokens passes dh_last[s] to
    dh0[s] unchanged.
    """
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    n = cu.size - 1
    T, W = np.shape(x)
    out = {k: np.zeros((T, W)) for k in ("dx", "dgx", "dga")}
    out["dlam"] = np.zeros(W)
    out["dh0"] = np.zeros((n, W)) if dh_last is None else _f64(dh_last).copy()
    for k in range(n):
        lo, hi = int(cu[k]), int(cu[k + 1])
        if hi <= lo:
            continue
        sl = slice(lo, hi)
        g = rglru_backward(_f64(x)[None, sl], _f64(gx)[None, sl], _f64(ga)[None, sl], lam, _f64(dh)[None, sl],
                           None if reset is None else np.asarray(reset)[None, sl],
                           None if h0 is None else _f64(h0)[k][None],
                           None if dh_last is None else _f64(dh_last)[k][None], c)
        for name in ("dx", "dgx", "dga"):
            out[name][sl] = g[name][0]
        out["dlam"] += g["dlam"]
        out["dh0"][k] = g["dh0"][0]
    return out


def rglru_forward_chunked(x, gx, ga, lam, reset=None, h0=None, c=C_DEFAULT, chunk=64):
    """The same forward, composed from per-chunk affine maps (exact, not approximate).

    The Fattori comparison page credits its authors with an exact parallel
    chunk forward with partial chunks. Each chunk of `chunk` steps (the last
    may be shorter) is reduced to a map h_in -> R ? B : A*h_in + B, where R
    records a reset inside the chunk; an exclusive scan over the chunks gives
    each chunk's incoming state; a replay of each chunk from that state gives h.
    """
    x = _f64(x)
    B, L, W = x.shape
    i, r, s, l, a, m = gates(gx, ga, lam, c)
    rst = _reset_mask(reset, B, L)
    alpha = np.where(rst[:, :, None], 0.0, a)
    u = np.where(rst[:, :, None], 1.0, m) * i * x
    n_chunks = -(-L // chunk)
    aggs = []
    for k in range(n_chunks):
        A = np.ones((B, W))
        Bv = np.zeros((B, W))
        R = np.zeros((B, 1), dtype=bool)
        for t in range(k * chunk, min(L, (k + 1) * chunk)):
            rt = rst[:, t][:, None]
            Bv = np.where(rt, u[:, t], alpha[:, t] * Bv + u[:, t])
            A = A * alpha[:, t]
            R = R | rt
        aggs.append((A, Bv, R))
    carry = np.zeros((B, W)) if h0 is None else _f64(h0).copy()
    starts = []
    for A, Bv, R in aggs:
        starts.append(carry)
        carry = np.where(R, Bv, A * carry + Bv)
    h = np.empty((B, L, W))
    for k in range(n_chunks):
        prev = starts[k]
        for t in range(k * chunk, min(L, (k + 1) * chunk)):
            rt = rst[:, t][:, None]
            prev = np.where(rt, u[:, t], alpha[:, t] * prev + u[:, t])
            h[:, t] = prev
    return h, carry


def blockdiag_proj_forward(x, w, b):
    """Block-diagonal linear map (the gate projections feeding the scan).

    x [T, W]; w [nb, bs, bs] read as [block, in, out]; b [W]. Output block k is
    x[:, k*bs:(k+1)*bs] @ w[k] + b[k*bs:(k+1)*bs].
    """
    x = _f64(x)
    w = _f64(w)
    T, W = x.shape
    nb, bs, _ = w.shape
    y = np.empty((T, W))
    for k in range(nb):
        sl = slice(k * bs, (k + 1) * bs)
        y[:, sl] = x[:, sl] @ w[k]
    return y + _f64(b)[None, :]


def blockdiag_proj_backward(x, w, dy):
    """Gradients of blockdiag_proj_forward: returns (dx [T, W], dw [nb, bs, bs], db [W])."""
    x = _f64(x)
    w = _f64(w)
    dy = _f64(dy)
    T, W = x.shape
    nb, bs, _ = w.shape
    dx = np.empty((T, W))
    dw = np.empty((nb, bs, bs))
    for k in range(nb):
        sl = slice(k * bs, (k + 1) * bs)
        dx[:, sl] = dy[:, sl] @ w[k].T
        dw[k] = x[:, sl].T @ dy[:, sl]
    return dx, dw, dy.sum(axis=0)
