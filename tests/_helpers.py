"""Shared test plumbing: moving synth inputs to the device, running both sides, tolerances.

Tolerances (stated for the hot path): outputs pass elementwise when
|got - ref| <= tol * max(1, |ref|), tol = 1e-5 for float32 io and 4e-3 for bf16
io; gradients pass per tensor when max|got - ref| <= tol * max(1, max|ref|),
tol = 1e-5 for float32 io and 1e-2 for bf16 io. The per-position gradients
(dx, dgate_x, dgate_a) must also pass elementwise, |got - ref| <=
tol * max(1, |ref|) with tol = 1e-4 for float32 io (the float32 reverse carry
accumulates up to L terms) and 1e-2 for bf16 io (one bf16 rounding of the
stored value is 2^-9 relative), so a small gradient next to a large one in the
same tensor is checked too.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synth

OUT_TOL = {"f32": 1e-5, "bf16": 4e-3}
GRAD_TOL = {"f32": 1e-5, "bf16": 1e-2}
GRAD_EL_TOL = {"f32": 1e-4, "bf16": 1e-2}


def to_dev(stored: synth.Stored, device="cuda") -> torch.Tensor:
    if stored.io == "f32":
        return torch.from_numpy(np.ascontiguousarray(stored.raw)).to(device)
    return torch.from_numpy(np.ascontiguousarray(stored.raw).view(np.int16)).view(torch.bfloat16).to(device)


def to_dev_f32(a, device="cuda"):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def to_dev_u8(a, device="cuda"):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(device)


def host64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


class DevInputs:
    """Device copies of one synth.Inputs."""

    def __init__(self, inp: synth.Inputs, device="cuda"):
        self.inp = inp
        self.x = to_dev(inp.x, device)
        self.gx = to_dev(inp.gx, device)
        self.ga = to_dev(inp.ga, device)
        self.dh = to_dev(inp.dh, device)
        self.lam = to_dev_f32(inp.lam, device)
        self.reset = to_dev_u8(inp.reset, device)
        self.h0 = to_dev_f32(inp.h0, device)
        self.dh_last = to_dev_f32(inp.dh_last, device)


def run_gpu(glr, d: DevInputs, chunk=None, want_bwd=True):
    wl = d.inp.wl
    chunk = wl.chunk if chunk is None else chunk
    h, h_last, ckpt = glr.rglru_fwd(d.x, d.gx, d.ga, d.lam, d.reset, d.h0, chunk=chunk)
    out = {"h": h, "h_last": h_last}
    if want_bwd:
        dx, dgx, dga, dlam, dh0 = glr.rglru_bwd(d.x, d.gx, d.ga, d.lam, d.reset, ckpt, d.dh, d.dh_last,
                                                chunk=chunk, want_dh0=True)
        out.update(dx=dx, dgx=dgx, dga=dga, dlam=dlam, dh0=dh0)
    torch.cuda.synchronize()
    return out


def run_oracle(inp: synth.Inputs, chans=None, want_bwd=True):
    """Oracle on all channels, or on the channel subset `chans` (channels are independent)."""
    sl = slice(None) if chans is None else np.asarray(chans)
    x = inp.x.value[:, :, sl]
    gx = inp.gx.value[:, :, sl]
    ga = inp.ga.value[:, :, sl]
    lam = inp.lam.astype(np.float64)[sl]
    h0 = None if inp.h0 is None else inp.h0.astype(np.float64)[:, sl]
    h, h_last = oracle.rglru_forward(x, gx, ga, lam, inp.reset, h0)
    out = {"h": h, "h_last": h_last}
    if want_bwd:
        dh = inp.dh.value[:, :, sl]
        dhl = None if inp.dh_last is None else inp.dh_last.astype(np.float64)[:, sl]
        out.update(oracle.rglru_backward(x, gx, ga, lam, dh, inp.reset, h0, dhl))
    return out


def out_err(got: np.ndarray, ref: np.ndarray) -> float:
    """Largest |got - ref| / max(1, |ref|)."""
    return float(np.max(np.abs(got - ref) / np.maximum(1.0, np.abs(ref)))) if ref.size else 0.0


def grad_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max|got - ref| / max(1, max|ref|)."""
    if ref.size == 0:
        return 0.0
    return float(np.max(np.abs(got - ref)) / max(1.0, float(np.max(np.abs(ref)))))


def compare(io: str, gpu: dict, ref: dict, chans=None, label=""):
    """Asserts every available output within tolerance; returns the error table."""
    sl = slice(None) if chans is None else np.asarray(chans)
    errs = {}
    errs["h"] = out_err(host64(gpu["h"])[:, :, sl], ref["h"])
    if gpu.get("h_last") is not None:
        errs["h_last"] = out_err(host64(gpu["h_last"])[:, sl], ref["h_last"])
    el = {}
    for k, rk in (("dx", "dx"), ("dgx", "dgx"), ("dga", "dga")):
        if k in gpu:
            g = host64(gpu[k])[:, :, sl]
            errs[k] = grad_err(g, ref[rk])
            el[k] = out_err(g, ref[rk])
    if "dlam" in gpu:
        errs["dlam"] = grad_err(host64(gpu["dlam"])[sl], ref["dlam"])
    if gpu.get("dh0") is not None:
        errs["dh0"] = grad_err(host64(gpu["dh0"])[:, sl], ref["dh0"])
    bad = {}
    for k, e in errs.items():
        tol = OUT_TOL[io] if k in ("h", "h_last") else GRAD_TOL[io]
        if not (e <= tol):
            bad[k] = (e, tol)
    for k, e in el.items():
        if not (e <= GRAD_EL_TOL[io]):
            bad[k + " (elementwise)"] = (e, GRAD_EL_TOL[io])
    assert not bad, f"{label} out of tolerance: {bad} (all errors: {errs}, elementwise: {el})"
    return errs


def sample_channels(W: int, n: int = 48, seed: int = 0) -> np.ndarray:
    """Spread channels plus the strip edges of every vector width the kernels use."""
    rng = np.random.default_rng(seed)
    edges = [0, 1, 63, 64, 127, 128, 255, 256, 511, 512, W - 1]
    ch = set(e for e in edges if 0 <= e < W)
    ch.update(rng.choice(W, size=min(n, W), replace=False).tolist())
    return np.array(sorted(ch))
