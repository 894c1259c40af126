"""Seeded synthetic inputs for the gated delta rule (GDN and KDA) workloads.

Input generation only, shared by the tests, the benchmark and the smoke
check: none of the recurrence's arithmetic lives here. q and k are drawn
N(0, 1) and scaled to unit length per token and head (the linear_attention
reference page takes its inputs already normalized), v is N(0, 1), beta is
sigmoid of an N(0, 1) draw, and the natural-log decay g has exp(g) ~ U[lo, hi]
(one value per value head for GDN, one per key channel for KDA). q, k, v are
stored in the io dtype (bf16 rounded to nearest even), g, beta and states in
float32. Both sides read the same stored values.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

from . import Stored, generator, store

# tensor ids inside a seed sequence (disjoint from the RG-LRU ids by the workload id)
D_Q, D_K, D_V, D_G, D_BETA, D_H0, D_LEN = range(7)


@dataclasses.dataclass(frozen=True)
class DeltaWorkload:
    wid: int
    name: str
    batch: int
    length: int
    k_heads: int
    v_heads: int
    k_dim: int
    v_dim: int
    io: str = "bf16"
    kda: bool = False
    decay_lo: float = 0.9
    decay_hi: float = 0.999
    h0: bool = False

    def resized(self, **kw) -> "DeltaWorkload":
        return dataclasses.replace(self, **kw)

    @property
    def tokens(self) -> int:
        return self.batch * self.length


DELTA_WORKLOADS = {
    # prefill at the RG-LRU workloads' batch and length, 16 heads of 128 x 128 state
    10: DeltaWorkload(10, "gdn_b4_t2048_h16_d128", 4, 2048, 16, 16, 128, 128),
    11: DeltaWorkload(11, "kda_b4_t2048_h16_d128", 4, 2048, 16, 16, 128, 128, kda=True),
    # one decode step of 64 sequences from a nonzero state
    12: DeltaWorkload(12, "gdn_decode_b64_h16_d128", 64, 1, 16, 16, 128, 128, h0=True),
}


@dataclasses.dataclass
class DeltaInputs:
    wl: DeltaWorkload
    q: Stored                        # [B, T, Hk, Dk]
    k: Stored                        # [B, T, Hk, Dk]
    v: Stored                        # [B, T, Hv, Dv]
    g: np.ndarray                    # float32 [B, T, Hv] (GDN) or [B, T, Hv, Dk] (KDA)
    beta: np.ndarray                 # float32 [B, T, Hv]
    h0: Optional[np.ndarray]         # float32 [N, Hv, Dk, Dv] or None
    cu: Optional[np.ndarray] = None  # int32 [N + 1] for packed sequences (B = 1)


def _unit(wid, tensor, shape, io, variant) -> Stored:
    a = generator(wid, tensor, variant).standard_normal(shape)
    return store(a / np.linalg.norm(a, axis=-1, keepdims=True), io)


def make_delta_inputs(wl: DeltaWorkload, variant: int = 0, lengths=None) -> DeltaInputs:
    """Inputs of wl; with lengths, one packed row (B = 1) of sequences of those lengths."""
    cu = None
    B, T = wl.batch, wl.length
    if lengths is not None:
        lengths = np.asarray(lengths, dtype=np.int64)
        cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
        B, T = 1, int(cu[-1])
    wid = wl.wid
    q = _unit(wid, D_Q, (B, T, wl.k_heads, wl.k_dim), wl.io, variant)
    k = _unit(wid, D_K, (B, T, wl.k_heads, wl.k_dim), wl.io, variant)
    v = store(generator(wid, D_V, variant).standard_normal((B, T, wl.v_heads, wl.v_dim)), wl.io)
    gshape = (B, T, wl.v_heads, wl.k_dim) if wl.kda else (B, T, wl.v_heads)
    g = np.log(generator(wid, D_G, variant).uniform(wl.decay_lo, wl.decay_hi, gshape)).astype(np.float32)
    z = generator(wid, D_BETA, variant).standard_normal((B, T, wl.v_heads))
    beta = (1.0 / (1.0 + np.exp(-z))).astype(np.float32)
    n = B if cu is None else len(cu) - 1
    h0 = None
    if wl.h0:
        h0 = generator(wid, D_H0, variant).standard_normal((n, wl.v_heads, wl.k_dim, wl.v_dim)).astype(np.float32)
    return DeltaInputs(wl, q, k, v, g, beta, h0, cu)


def seq_lengths(n, mean, variant=0, empty_p=0.0) -> np.ndarray:
    """n lengths, Geometric(1/mean), each made empty with probability empty_p."""
    g = generator(92, D_LEN, variant)
    lens = g.geometric(1.0 / mean, size=n).astype(np.int64)
    lens[g.random(n) < empty_p] = 0
    return lens
