"""Seeded synthetic inputs for the RG-LRU scan workloads.

This module is shared by the tests, the benchmark and the smoke check. It holds
input generation only: random draws, the bf16 rounding of stored values, the
document/reset layout and the per-channel decay parameter. None of the
recurrence's arithmetic lives here; the oracle and the HIP path each compute
the method on their own from what this module hands them.

Every draw comes from numpy's PCG64 seeded by SeedSequence([workload, tensor,
variant]), is made in float64, cast to float32, and (for bf16 tensors) rounded
to bf16 by round-to-nearest-even. Both sides read the same stored values.

Workloads mirror the shapes and distributions of the pages' benchmark
(Fattori comparison JSON page: shape block B=4, L=2048, W=2048, BF16 with an
FP32 carry) and the four companion cases of the hot-path scope.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

# tensor ids inside a seed sequence
T_X, T_GX, T_GA, T_LAM, T_DH, T_H0, T_RESET, T_WX, T_WA, T_DHLAST, T_SEQLEN = range(11)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: shape, io dtype and input distributions."""
    wid: int
    name: str
    batch: int
    length: int
    width: int
    io: str                      # "f32" or "bf16"
    decay_lo: float              # exp(-8*softplus(lam)) ~ U[decay_lo, decay_hi]
    decay_hi: float
    doc_mean: Optional[float]    # mean document length (None: no resets)
    h0: bool                     # nonzero FP32 initial state with gradient
    chunk: int = 0               # time-chunk of the parallel scan (0: library default)
    proj_blocks: int = 0         # block-diagonal gate projection blocks (0: none)
    proj_block: int = 256

    @property
    def elems(self) -> int:
        return self.batch * self.length * self.width

    def resized(self, batch=None, length=None, width=None, chunk=None,
                proj_blocks=None, proj_block=None) -> "Workload":
        return dataclasses.replace(
            self,
            batch=self.batch if batch is None else batch,
            length=self.length if length is None else length,
            width=self.width if width is None else width,
            chunk=self.chunk if chunk is None else chunk,
            proj_blocks=self.proj_blocks if proj_blocks is None else proj_blocks,
            proj_block=self.proj_block if proj_block is None else proj_block,
        )


WORKLOADS = {
    0: Workload(0, "tiny_f32", 1, 64, 64, "f32", 0.9, 0.999, None, False),
    1: Workload(1, "restricted_b4_l2048_w2048", 4, 2048, 2048, "bf16", 0.9, 0.999, None, False),
    2: Workload(2, "canonical_reset_b4_l2048_w2048", 4, 2048, 2048, "bf16", 0.9, 0.999, 512.0, True),
    3: Workload(3, "long_b1_l32768_w4096", 1, 32768, 4096, "bf16", 0.99, 0.9999, 4096.0, True,
                chunk=256),
    4: Workload(4, "blockdiag_b8_l4096_w2560", 8, 4096, 2560, "bf16", 0.9, 0.999, 1024.0, True,
                proj_blocks=10, proj_block=256),
    # the pages' measured scope at their shape: both gate projections (8
    # blocks of 256, an assumed block count) and the scan, restricted contract
    5: Workload(5, "restricted_proj_b4_l2048_w2048", 4, 2048, 2048, "bf16", 0.9, 0.999, None, False,
                proj_blocks=8, proj_block=256),
}


def generator(wid: int, tensor: int, variant: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([wid, tensor, variant])))


# ---------------------------------------------------------------- bf16 storage

def f32_to_bf16_bits(a) -> np.ndarray:
    """Round float32 values to bf16 (round-to-nearest-even); returns uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    out[nan] = ((u[nan] >> 16) | 0x0040).astype(np.uint16)   # keep sign, force quiet
    return out


def bf16_bits_to_f32(bits) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class Stored:
    """A tensor as stored for the device (f32 array or bf16 bit pattern) plus its exact value."""
    io: str
    raw: np.ndarray          # float32, or uint16 bf16 bits
    value: np.ndarray        # float64, exactly the stored value

    @property
    def shape(self):
        return self.raw.shape


def store(values_f64: np.ndarray, io: str) -> Stored:
    f32 = np.asarray(values_f64, dtype=np.float64).astype(np.float32)
    if io == "f32":
        return Stored(io, f32, f32.astype(np.float64))
    if io == "bf16":
        bits = f32_to_bf16_bits(f32)
        return Stored(io, bits, bf16_bits_to_f32(bits).astype(np.float64))
    raise ValueError(io)


# ---------------------------------------------------------------- draws

def normal(wid, tensor, shape, io, variant=0, scale=1.0) -> Stored:
    return store(generator(wid, tensor, variant).standard_normal(shape) * scale, io)


def decay_param(wid, width, lo, hi, variant=0) -> np.ndarray:
    """Per-channel float32 lambda with exp(-8*softplus(lambda)) ~ U[lo, hi].

    The target decay u gives softplus(lambda) = -ln(u)/8, so lambda is the
    inverse softplus of that value, log(expm1(y)). This is how the input is
    drawn, not part of the recurrence.
    """
    u = generator(wid, T_LAM, variant).uniform(lo, hi, size=width)
    y = -np.log(u) / 8.0
    return np.log(np.expm1(y)).astype(np.float32)


def reset_flags(wid, batch, length, doc_mean, variant=0) -> np.ndarray:
    """uint8 [B, L]: 1 marks the first token of a document.

    Each row continues a document carried in by the initial state, so the first
    reset lands at an offset drawn from Geometric(1/doc_mean) (support 1, 2, ...);
    every later document has a Geometric(1/doc_mean) length.
    """
    g = generator(wid, T_RESET, variant)
    p = 1.0 / doc_mean
    flags = np.zeros((batch, length), dtype=np.uint8)
    for b in range(batch):
        pos = int(g.geometric(p))
        while pos < length:
            flags[b, pos] = 1
            pos += int(g.geometric(p))
    return flags


@dataclasses.dataclass
class Inputs:
    wl: Workload
    x: Stored
    gx: Stored
    ga: Stored
    lam: np.ndarray                 # float32 [W]
    dh: Stored
    reset: Optional[np.ndarray]     # uint8 [B, L] or None
    h0: Optional[np.ndarray]        # float32 [B, W] or None
    dh_last: Optional[np.ndarray]   # float32 [B, W] or None
    wx: Optional[Stored] = None     # bf16 [nb, bs, bs] (in, out)
    wa: Optional[Stored] = None
    bx: Optional[Stored] = None     # bf16 [W] zeros
    ba: Optional[Stored] = None


def make_inputs(wl: Workload, variant: int = 0, with_dh_last: bool = False,
                force_reset0: bool = False) -> Inputs:
    """All inputs of one workload, drawn from its seeds."""
    B, L, W, io = wl.batch, wl.length, wl.width, wl.io
    shape = (B, L, W)
    x = normal(wl.wid, T_X, shape, io, variant)
    gx = normal(wl.wid, T_GX, shape, io, variant)
    ga = normal(wl.wid, T_GA, shape, io, variant)
    dh = normal(wl.wid, T_DH, shape, io, variant)
    lam = decay_param(wl.wid, W, wl.decay_lo, wl.decay_hi, variant)
    reset = None
    if wl.doc_mean is not None:
        reset = reset_flags(wl.wid, B, L, wl.doc_mean, variant)
    if force_reset0:
        if reset is None:
            reset = np.zeros((B, L), dtype=np.uint8)
        reset[:, 0] = 1
    h0 = None
    if wl.h0:
        h0 = generator(wl.wid, T_H0, variant).standard_normal((B, W)).astype(np.float32)
    dh_last = None
    if with_dh_last:
        dh_last = generator(wl.wid, T_DHLAST, variant).standard_normal((B, W)).astype(np.float32)
    inp = Inputs(wl, x, gx, ga, lam, dh, reset, h0, dh_last)
    if wl.proj_blocks:
        nb, bs = wl.proj_blocks, wl.proj_block
        if nb * bs != W:
            raise ValueError("projection blocks must tile the width")
        sd = 1.0 / math.sqrt(bs)
        inp.wx = normal(wl.wid, T_WX, (nb, bs, bs), "bf16", variant, scale=sd)
        inp.wa = normal(wl.wid, T_WA, (nb, bs, bs), "bf16", variant, scale=sd)
        inp.bx = store(np.zeros(W), "bf16")
        inp.ba = store(np.zeros(W), "bf16")
    return inp


# ---------------------------------------------------------------- packed sequences

@dataclasses.dataclass
class VarlenInputs:
    """Packed sequences: [T, W] tensors, offsets cu [n + 1], per-sequence states [n, W]."""
    io: str
    cu: np.ndarray                  # int32 [n + 1]
    x: Stored
    gx: Stored
    ga: Stored
    lam: np.ndarray                 # float32 [W]
    dh: Stored
    reset: Optional[np.ndarray]     # uint8 [T] or None
    h0: Optional[np.ndarray]        # float32 [n, W] or None
    dh_last: Optional[np.ndarray]   # float32 [n, W] or None


def seq_lengths(n, mean, variant=0, empty_p=0.0) -> np.ndarray:
    """n sequence lengths, Geometric(1/mean) (support 1, 2, ...), each made empty with probability empty_p."""
    g = generator(90, T_SEQLEN, variant)
    lens = g.geometric(1.0 / mean, size=n).astype(np.int64)
    lens[g.random(n) < empty_p] = 0
    return lens


def make_varlen_inputs(lengths, width, io, variant=0, decay=(0.9, 0.999), reset_mean=None,
                       with_h0=True, with_dh_last=True) -> VarlenInputs:
    """Inputs of packed sequences with the given lengths (total at least 1 token)."""
    lengths = np.asarray(lengths, dtype=np.int64)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T, n, W = int(cu[-1]), lengths.size, width
    wid = 91
    x = normal(wid, T_X, (T, W), io, variant)
    gx = normal(wid, T_GX, (T, W), io, variant)
    ga = normal(wid, T_GA, (T, W), io, variant)
    dh = normal(wid, T_DH, (T, W), io, variant)
    lam = decay_param(wid, W, decay[0], decay[1], variant)
    reset = None
    if reset_mean is not None:
        reset = reset_flags(wid, 1, T, reset_mean, variant)[0]
    h0 = generator(wid, T_H0, variant).standard_normal((n, W)).astype(np.float32) if with_h0 else None
    dhl = generator(wid, T_DHLAST, variant).standard_normal((n, W)).astype(np.float32) if with_dh_last else None
    return VarlenInputs(io, cu, x, gx, ga, lam, dh, reset, h0, dhl)
