"""Float64 CPU oracle of the gated delta rule (GDN: a scalar decay per value
head; KDA: a decay per key channel).

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import or run this module. The product path (the HIP
library and its Python binding) never calls it and shares no code with it.

The linear_attention reference page (modelopt.torch.quantization
.linear_attention.reference) gives the two oracles this mirrors by name,
signature and shapes: q, k [B, T, Hk, Dk]; v [B, T, Hv, Dv]; beta [B, T, Hv];
g [B, T, Hv] (GDN) or [B, T, Hv, Dk] (KDA), natural-log gates; state
[N, Hv, Dk, Dv] (key-first) or [N, Hv, Dv, Dk] (state_v_first); packed
sequences through cu_seqlens (then B = 1 and N sequences); output and final
state returned; the chunk form is exact algebra around a unit-lower-triangular
solve. It does not print the recurrence. The readings taken here (each also
listed with the other readings of the pages):

  per value head h (key head h // (Hv / Hk)), per token t, S the [Dk, Dv] state:
    S <- diag(exp(g_t)) S            (GDN: exp(g_t) times S)
    S <- S + k_t (beta_t (v_t - S^T k_t))^T
    o_t = scale * S^T q_t,  scale = 1 / sqrt(Dk) unless given
  S starts from the sequence's initial state (zeros if none). q and k are
  used as given (the page: inputs arrive normalized/activated).

Arithmetic is float64 on the given values; nothing is rounded. Pinned by
tests/test_oracle_delta.py against closed forms (no write: pure decay; unit
writes of orthogonal keys: exact recall and overwrite), a hand-derived
two-token example, the two forms against each other, and layout identities.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.linalg import solve_triangular


def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def _sequences(B, T, cu_seqlens):
    """(batch row, first token, end token) of each sequence."""
    if cu_seqlens is None:
        return [(b, 0, T) for b in range(B)]
    if B != 1:
        raise ValueError("packed sequences need B = 1")
    cu = [int(c) for c in cu_seqlens]
    if cu[0] != 0 or cu[-1] != T or any(cu[i] > cu[i + 1] for i in range(len(cu) - 1)):
        raise ValueError("cu_seqlens must rise from 0 to T")
    return [(0, cu[n], cu[n + 1]) for n in range(len(cu) - 1)]


def _heads(q, v):
    B, T, Hk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    if Hv % Hk != 0:
        raise ValueError("Hv must be a multiple of Hk")
    return B, T, Hk, Dk, Hv, Dv, Hv // Hk


def recurrent_delta_rule(q, k, v, g, beta, scale=None, initial_state=None, cu_seqlens=None,
                         state_v_first=False):
    """Token-by-token gated delta rule (GDN when g is [B, T, Hv], KDA when [B, T, Hv, Dk]).
    Returns (o [B, T, Hv, Dv], final state [N, Hv, Dk, Dv] or [N, Hv, Dv, Dk])."""
    q, k, v, g, beta = (_f64(a) for a in (q, k, v, g, beta))
    B, T, Hk, Dk, Hv, Dv, grp = _heads(q, v)
    kda = g.ndim == 4
    sc = 1.0 / math.sqrt(Dk) if scale is None else float(scale)
    seqs = _sequences(B, T, cu_seqlens)
    h0 = _f64(initial_state)
    o = np.zeros((B, T, Hv, Dv))
    fin = np.zeros((len(seqs), Hv, Dk, Dv))
    for n, (b, s0, s1) in enumerate(seqs):
        for h in range(Hv):
            kh = h // grp
            if h0 is None:
                S = np.zeros((Dk, Dv))
            else:
                S = (h0[n, h].T if state_v_first else h0[n, h]).copy()
            for t in range(s0, s1):
                if kda:
                    S = np.exp(g[b, t, h])[:, None] * S
                else:
                    S = np.exp(g[b, t, h]) * S
                kt = k[b, t, kh]
                u = beta[b, t, h] * (v[b, t, h] - S.T @ kt)
                S = S + np.outer(kt, u)
                o[b, t, h] = sc * (S.T @ q[b, t, kh])
            fin[n, h] = S
    if state_v_first:
        fin = fin.transpose(0, 1, 3, 2)
    return o, fin


def chunk_gdn(q, k, v, g, beta, chunk_size=64, scale=None, initial_state=None, cu_seqlens=None,
              state_v_first=False):
    """The same GDN recurrence (scalar decay per value head) in chunk form.

    Within a chunk of n tokens, with Gc_i the running sum of the chunk's log
    decays up to token i, S0 the state entering the chunk and u_i the
    corrected write of token i (u_i = beta_i (v_i - S_{i-1}^T k_i), S_{i-1}
    already decayed to step i):

        u_i = beta_i v_i - beta_i e^{Gc_i} (S0^T k_i)
              - sum_{j<i} beta_i e^{Gc_i - Gc_j} (k_i . k_j) u_j,

    so (I + A) U = diag(beta) V - diag(beta e^{Gc}) K S0 with A the strictly
    lower matrix A_ij = beta_i e^{Gc_i - Gc_j} k_i . k_j: one unit-lower-
    triangular solve per chunk. Then

        o_i   = scale (e^{Gc_i} q_i^T S0 + sum_{j<=i} e^{Gc_i - Gc_j} (q_i . k_j) u_j)
        S_end = e^{Gc_last} S0 + sum_j e^{Gc_last - Gc_j} k_j u_j^T.
    """
    q, k, v, g, beta = (_f64(a) for a in (q, k, v, g, beta))
    if g.ndim != 3:
        raise ValueError("chunk_gdn takes the scalar (GDN) decay [B, T, Hv]")
    B, T, Hk, Dk, Hv, Dv, grp = _heads(q, v)
    sc = 1.0 / math.sqrt(Dk) if scale is None else float(scale)
    seqs = _sequences(B, T, cu_seqlens)
    h0 = _f64(initial_state)
    o = np.zeros((B, T, Hv, Dv))
    fin = np.zeros((len(seqs), Hv, Dk, Dv))
    for n, (b, s0, s1) in enumerate(seqs):
        for h in range(Hv):
            kh = h // grp
            if h0 is None:
                S = np.zeros((Dk, Dv))
            else:
                S = (h0[n, h].T if state_v_first else h0[n, h]).copy()
            for c0 in range(s0, s1, chunk_size):
                c1 = min(c0 + chunk_size, s1)
                K = k[b, c0:c1, kh]
                Q = q[b, c0:c1, kh]
                V = v[b, c0:c1, h]
                be = beta[b, c0:c1, h]
                Gc = np.cumsum(g[b, c0:c1, h])
                D = np.exp(Gc[:, None] - Gc[None, :])          # e^{Gc_i - Gc_j}
                A = np.tril(be[:, None] * D * (K @ K.T), -1)
                rhs = be[:, None] * V - (be * np.exp(Gc))[:, None] * (K @ S)
                U = solve_triangular(np.eye(c1 - c0) + A, rhs, lower=True, unit_diagonal=True)
                o[b, c0:c1, h] = sc * (np.exp(Gc)[:, None] * (Q @ S) + np.tril(D * (Q @ K.T)) @ U)
                S = np.exp(Gc[-1]) * S + (np.exp(Gc[-1] - Gc)[:, None] * K).T @ U
            fin[n, h] = S
    if state_v_first:
        fin = fin.transpose(0, 1, 3, 2)
    return o, fin


def recurrent_delta_rule_backward(q, k, v, g, beta, do, dh_last=None, scale=None, initial_state=None,
                                  cu_seqlens=None, state_v_first=False):
    """Gradients of the token recurrence above for the loss <do, o> + <dh_last, S_final>.

    Reverse-mode differentiation of each step, written out (the page's oracles keep autograd
    gradients, through the initial state included). With S~ = D S_prev (the decayed state),
    e = v - S~^T k, u = beta e, S = S~ + k u^T, o = scale S^T q, and G the gradient of S:
      G += scale q do^T;  dq = scale S do;  du = G^T k;  dv = beta du;  dbeta = e . du;
      G~ = G - beta k du^T  (gradient of S~);  dk = G u - beta S~ du;
      dg = <G~, S~> (GDN) or the row sums of G~ * S~ (KDA);  G <- D G~ for the step before.
    Returns (dq, dk, dv, dg, dbeta, dh0) with the shapes of q, k, v, g, beta and the states.
    """
    q, k, v, g, beta, do = (_f64(a) for a in (q, k, v, g, beta, do))
    B, T, Hk, Dk, Hv, Dv, grp = _heads(q, v)
    kda = g.ndim == 4
    sc = 1.0 / math.sqrt(Dk) if scale is None else float(scale)
    seqs = _sequences(B, T, cu_seqlens)
    h0 = _f64(initial_state)
    dhl = _f64(dh_last)
    dq, dk = np.zeros_like(q), np.zeros_like(k)
    dv, dg, dbeta = np.zeros_like(v), np.zeros_like(g), np.zeros_like(beta)
    dh0 = np.zeros((len(seqs), Hv, Dk, Dv))
    for n, (b, s0, s1) in enumerate(seqs):
        for h in range(Hv):
            kh = h // grp
            if h0 is None:
                S = np.zeros((Dk, Dv))
            else:
                S = (h0[n, h].T if state_v_first else h0[n, h]).copy()
            hist = []   # (S~, e, u) of every step, forward order
            for t in range(s0, s1):
                dec = np.exp(g[b, t, h])
                St = (dec[:, None] if kda else dec) * S
                kt = k[b, t, kh]
                e = v[b, t, h] - St.T @ kt
                u = beta[b, t, h] * e
                S = St + np.outer(kt, u)
                hist.append((St, e, u))
            if dhl is None:
                G = np.zeros((Dk, Dv))
            else:
                G = (dhl[n, h].T if state_v_first else dhl[n, h]).copy()
            for t in range(s1 - 1, s0 - 1, -1):
                St, e, u = hist[t - s0]
                kt, qt, dot = k[b, t, kh], q[b, t, kh], do[b, t, h]
                Sn = St + np.outer(kt, u)
                G = G + sc * np.outer(qt, dot)
                dq[b, t, kh] += sc * (Sn @ dot)
                du = G.T @ kt
                bt = beta[b, t, h]
                dv[b, t, h] = bt * du
                dbeta[b, t, h] = e @ du
                dk[b, t, kh] += G @ u - bt * (St @ du)
                Gt = G - bt * np.outer(kt, du)
                if kda:
                    dg[b, t, h] = np.sum(Gt * St, axis=1)
                    G = np.exp(g[b, t, h])[:, None] * Gt
                else:
                    dg[b, t, h] = np.sum(Gt * St)
                    G = np.exp(g[b, t, h]) * Gt
            dh0[n, h] = G
    if state_v_first:
        dh0 = dh0.transpose(0, 1, 3, 2)
    return dq, dk, dv, dg, dbeta, dh0
