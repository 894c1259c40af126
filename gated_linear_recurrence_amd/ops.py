"""Python binding of the C ABI, with the same entry-point names.

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, outputs are allocated with torch when the caller passes none, and
the raw pointers go to librglru. Every step of the computation runs in the
HIP kernels; nothing here computes.
"""
from __future__ import annotations

import ctypes
import weakref
from typing import Optional

import torch

from . import _lib

_IO = {torch.float32: _lib.RGLRU_IO_F32, torch.bfloat16: _lib.RGLRU_IO_BF16}


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, shape, dtype, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _opt(t, name, shape, dtype, device):
    return None if t is None else _need(t, name, shape, dtype, device)


def make_shape(batch, length, width, io_dtype, chunk=0, c=8.0) -> _lib.rglru_shape_t:
    io = _IO[io_dtype] if isinstance(io_dtype, torch.dtype) else int(io_dtype)
    return _lib.rglru_shape_t(int(batch), int(length), int(width), io, int(chunk), float(c), 0)


def rglru_ckpt_elems(shape: _lib.rglru_shape_t) -> int:
    return int(_lib.load().rglru_ckpt_elems(ctypes.byref(shape)))


def rglru_fwd_workspace_bytes(shape: _lib.rglru_shape_t) -> int:
    return int(_lib.load().rglru_fwd_workspace_bytes(ctypes.byref(shape)))


def rglru_bwd_workspace_bytes(shape: _lib.rglru_shape_t) -> int:
    return int(_lib.load().rglru_bwd_workspace_bytes(ctypes.byref(shape)))


def rglru_workspace_bytes(shape: _lib.rglru_shape_t) -> int:
    return int(_lib.load().rglru_workspace_bytes(ctypes.byref(shape)))


class Workspace:
    """A zero-initialised device buffer reused by consecutive calls on one stream.

    The library leaves it ready for the next call after each one, so it is
    zero-filled only when (re)allocated. Calls sharing one Workspace must not
    overlap in time.
    """

    def __init__(self, device=None):
        self.device = torch.device(device if device is not None else "cuda")
        self.buf = None
        _workspaces.add(self)

    def get(self, nbytes: int) -> torch.Tensor:
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=self.device)
        return self.buf

    def error_bits(self) -> int:
        """Sticky error word of the header (synchronises with the device).

        Bit 0: a wait for another workgroup's published prefix hit its spin
        limit. Bit 1: a wait between the waves of one workgroup hit its spin
        limit. Bit 2: the offsets of a packed-sequence call were not valid.
        Each invalidates the outputs of the call that set it.
        """
        if self.buf is None:
            return 0
        return int(self.buf[12:16].view(torch.int32).item()) & 0xFFFFFFFF

    def raise_if_error(self) -> None:
        """Raises WorkspaceError if any call on this workspace set an error bit."""
        bits = self.error_bits()
        if bits:
            raise WorkspaceError(bits)

    def clear_errors(self) -> None:
        """Zeroes the sticky error word (on the current stream)."""
        if self.buf is not None:
            self.buf[12:16].zero_()


class WorkspaceError(RuntimeError):
    """A scan's bounded wait ran out: the outputs of that call are invalid."""

    def __init__(self, bits: int):
        kinds = []
        if bits & 1:
            kinds.append("cross-workgroup look-back wait hit its spin limit")
        if bits & 2:
            kinds.append("wait between waves of a workgroup hit its spin limit")
        if bits & 4:
            kinds.append("packed-sequence offsets (cu_seqlens) were not valid")
        if bits & ~7:
            kinds.append(f"unknown bits {bits & ~7:#x}")
        super().__init__("rglru workspace error word %#x: %s" % (bits, "; ".join(kinds)))
        self.bits = bits


_workspaces = weakref.WeakSet()


def check_errors() -> None:
    """Raises WorkspaceError if any live workspace (the defaults included) holds an error bit."""
    for ws in list(_workspaces):
        ws.raise_if_error()


_default_ws = {}


def default_workspace(device: torch.device) -> Workspace:
    key = (device.index, torch.cuda.current_stream(device).cuda_stream)
    ws = _default_ws.get(key)
    if ws is None:
        ws = _default_ws[key] = Workspace(device)
    return ws


def rglru_fwd(x: torch.Tensor, gate_x: torch.Tensor, gate_a: torch.Tensor, lam: torch.Tensor,
              reset: Optional[torch.Tensor] = None, h0: Optional[torch.Tensor] = None, *,
              chunk: int = 0, c: float = 8.0, training: bool = True, want_h_last: bool = True,
              h: Optional[torch.Tensor] = None, h_last: Optional[torch.Tensor] = None,
              ckpt: Optional[torch.Tensor] = None, workspace: Optional[Workspace] = None):
    """Forward scan. Returns (h, h_last or None, ckpt or None)."""
    lib = _lib.load()
    dev = x.device
    if x.dim() != 3:
        raise ValueError("x must be [B, L, W]")
    B, L, W = x.shape
    io = x.dtype
    if io not in _IO:
        raise ValueError(f"unsupported io dtype {io}")
    _need(x, "x", (B, L, W), io, dev)
    _need(gate_x, "gate_x", (B, L, W), io, dev)
    _need(gate_a, "gate_a", (B, L, W), io, dev)
    _need(lam, "lambda", (W,), torch.float32, dev)
    _opt(reset, "reset", (B, L), torch.uint8, dev)
    _opt(h0, "h0", (B, W), torch.float32, dev)
    shape = make_shape(B, L, W, io, chunk, c)
    if h is None:
        h = torch.empty((B, L, W), dtype=io, device=dev)
    _need(h, "h", (B, L, W), io, dev)
    if h_last is None and want_h_last:
        h_last = torch.empty((B, W), dtype=torch.float32, device=dev)
    _opt(h_last, "h_last", (B, W), torch.float32, dev)
    if ckpt is None and training:
        ckpt = torch.empty(rglru_ckpt_elems(shape), dtype=torch.float32, device=dev)
    if ckpt is not None:
        _need(ckpt, "ckpt", (rglru_ckpt_elems(shape),), torch.float32, dev)
    ws = workspace if workspace is not None else default_workspace(dev)
    nbytes = rglru_workspace_bytes(shape)
    buf = ws.get(nbytes)
    st = lib.rglru_fwd(ctypes.byref(shape), _ptr(x), _ptr(gate_x), _ptr(gate_a), _ptr(lam), _ptr(reset),
                       _ptr(h0), _ptr(h), _ptr(h_last), _ptr(ckpt), _ptr(buf), buf.numel(), _stream(dev))
    _lib.check(st, "rglru_fwd")
    return h, h_last, ckpt


def rglru_fwd_scratch(x: torch.Tensor, gate_x: torch.Tensor, gate_a: torch.Tensor, lam: torch.Tensor,
                      reset: Optional[torch.Tensor] = None, h0: Optional[torch.Tensor] = None, *,
                      h: torch.Tensor, h_last: Optional[torch.Tensor] = None, ckpt: Optional[torch.Tensor] = None,
                      chunk: int = 0, c: float = 8.0):
    """Forward scan through the allocation-free entry point: no workspace, and
    every output passed in (nothing is allocated here either). Returns (h,
    h_last, ckpt)."""
    lib = _lib.load()
    dev = x.device
    B, L, W = x.shape
    io = x.dtype
    if io not in _IO:
        raise ValueError(f"unsupported io dtype {io}")
    _need(x, "x", (B, L, W), io, dev)
    _need(gate_x, "gate_x", (B, L, W), io, dev)
    _need(gate_a, "gate_a", (B, L, W), io, dev)
    _need(lam, "lambda", (W,), torch.float32, dev)
    _opt(reset, "reset", (B, L), torch.uint8, dev)
    _opt(h0, "h0", (B, W), torch.float32, dev)
    _need(h, "h", (B, L, W), io, dev)
    _opt(h_last, "h_last", (B, W), torch.float32, dev)
    shape = make_shape(B, L, W, io, chunk, c)
    if ckpt is not None:
        _need(ckpt, "ckpt", (rglru_ckpt_elems(shape),), torch.float32, dev)
    st = lib.rglru_fwd_scratch(ctypes.byref(shape), _ptr(x), _ptr(gate_x), _ptr(gate_a), _ptr(lam), _ptr(reset),
                               _ptr(h0), _ptr(h), _ptr(h_last), _ptr(ckpt), _stream(dev))
    _lib.check(st, "rglru_fwd_scratch")
    return h, h_last, ckpt


def rglru_bwd(x: torch.Tensor, gate_x: torch.Tensor, gate_a: torch.Tensor, lam: torch.Tensor,
              reset: Optional[torch.Tensor], ckpt: torch.Tensor, dh: torch.Tensor,
              dh_last: Optional[torch.Tensor] = None, *, chunk: int = 0, c: float = 8.0,
              want_dh0: bool = True, dx: Optional[torch.Tensor] = None, dgate_x: Optional[torch.Tensor] = None,
              dgate_a: Optional[torch.Tensor] = None, dlam: Optional[torch.Tensor] = None,
              dh0: Optional[torch.Tensor] = None, workspace: Optional[Workspace] = None):
    """Backward scan. Returns (dx, dgate_x, dgate_a, dlambda, dh0 or None)."""
    lib = _lib.load()
    dev = x.device
    B, L, W = x.shape
    io = x.dtype
    if io not in _IO:
        raise ValueError(f"unsupported io dtype {io}")
    for t, n in ((x, "x"), (gate_x, "gate_x"), (gate_a, "gate_a"), (dh, "dh")):
        _need(t, n, (B, L, W), io, dev)
    _need(lam, "lambda", (W,), torch.float32, dev)
    _opt(reset, "reset", (B, L), torch.uint8, dev)
    _opt(dh_last, "dh_last", (B, W), torch.float32, dev)
    shape = make_shape(B, L, W, io, chunk, c)
    _need(ckpt, "ckpt", (rglru_ckpt_elems(shape),), torch.float32, dev)
    dx = torch.empty_like(x) if dx is None else _need(dx, "dx", (B, L, W), io, dev)
    dgate_x = torch.empty_like(x) if dgate_x is None else _need(dgate_x, "dgate_x", (B, L, W), io, dev)
    dgate_a = torch.empty_like(x) if dgate_a is None else _need(dgate_a, "dgate_a", (B, L, W), io, dev)
    dlam = torch.empty((W,), dtype=torch.float32, device=dev) if dlam is None else \
        _need(dlam, "dlambda", (W,), torch.float32, dev)
    if dh0 is None and want_dh0:
        dh0 = torch.empty((B, W), dtype=torch.float32, device=dev)
    _opt(dh0, "dh0", (B, W), torch.float32, dev)
    ws = workspace if workspace is not None else default_workspace(dev)
    nbytes = rglru_workspace_bytes(shape)
    buf = ws.get(nbytes)
    st = lib.rglru_bwd(ctypes.byref(shape), _ptr(x), _ptr(gate_x), _ptr(gate_a), _ptr(lam), _ptr(reset),
                       _ptr(ckpt), _ptr(dh), _ptr(dh_last), _ptr(dx), _ptr(dgate_x), _ptr(dgate_a),
                       _ptr(dlam), _ptr(dh0), _ptr(buf), buf.numel(), _stream(dev))
    _lib.check(st, "rglru_bwd")
    return dx, dgate_x, dgate_a, dlam, dh0


def rglru_varlen_workspace_bytes(shape: _lib.rglru_shape_t, n_seqs: int) -> int:
    return int(_lib.load().rglru_varlen_workspace_bytes(ctypes.byref(shape), int(n_seqs)))


def _varlen_common(x, gate_x, gate_a, lam, cu_seqlens, reset, h0):
    dev = x.device
    if x.dim() != 2:
        raise ValueError("packed x must be [T, W]")
    T, W = x.shape
    io = x.dtype
    if io not in _IO:
        raise ValueError(f"unsupported io dtype {io}")
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be [n + 1] with n >= 1")
    n = cu_seqlens.numel() - 1
    _need(cu_seqlens, "cu_seqlens", (n + 1,), torch.int32, dev)
    _need(x, "x", (T, W), io, dev)
    _need(gate_x, "gate_x", (T, W), io, dev)
    _need(gate_a, "gate_a", (T, W), io, dev)
    _need(lam, "lambda", (W,), torch.float32, dev)
    _opt(reset, "reset", (T,), torch.uint8, dev)
    _opt(h0, "h0", (n, W), torch.float32, dev)
    return dev, T, W, io, n


def rglru_fwd_varlen(x: torch.Tensor, gate_x: torch.Tensor, gate_a: torch.Tensor, lam: torch.Tensor,
                     cu_seqlens: torch.Tensor, reset: Optional[torch.Tensor] = None,
                     h0: Optional[torch.Tensor] = None, *, chunk: int = 0, c: float = 8.0, training: bool = True,
                     want_h_last: bool = True, h: Optional[torch.Tensor] = None,
                     h_last: Optional[torch.Tensor] = None, ckpt: Optional[torch.Tensor] = None,
                     workspace: Optional[Workspace] = None):
    """Forward scan of packed sequences: x [T, W], cu_seqlens [n + 1] int32 on the device.
    Returns (h [T, W], h_last [n, W] or None, ckpt or None)."""
    lib = _lib.load()
    dev, T, W, io, n = _varlen_common(x, gate_x, gate_a, lam, cu_seqlens, reset, h0)
    shape = make_shape(1, T, W, io, chunk, c)
    if h is None:
        h = torch.empty((T, W), dtype=io, device=dev)
    _need(h, "h", (T, W), io, dev)
    if h_last is None and want_h_last:
        h_last = torch.empty((n, W), dtype=torch.float32, device=dev)
    _opt(h_last, "h_last", (n, W), torch.float32, dev)
    if ckpt is None and training:
        ckpt = torch.empty(rglru_ckpt_elems(shape), dtype=torch.float32, device=dev)
    if ckpt is not None:
        _need(ckpt, "ckpt", (rglru_ckpt_elems(shape),), torch.float32, dev)
    ws = workspace if workspace is not None else default_workspace(dev)
    buf = ws.get(rglru_varlen_workspace_bytes(shape, n))
    st = lib.rglru_fwd_varlen(ctypes.byref(shape), _ptr(cu_seqlens), n, _ptr(x), _ptr(gate_x), _ptr(gate_a),
                              _ptr(lam), _ptr(reset), _ptr(h0), _ptr(h), _ptr(h_last), _ptr(ckpt), _ptr(buf),
                              buf.numel(), _stream(dev))
    _lib.check(st, "rglru_fwd_varlen")
    return h, h_last, ckpt


def rglru_bwd_varlen(x: torch.Tensor, gate_x: torch.Tensor, gate_a: torch.Tensor, lam: torch.Tensor,
                     cu_seqlens: torch.Tensor, reset: Optional[torch.Tensor], h0: Optional[torch.Tensor],
                     ckpt: torch.Tensor, dh: torch.Tensor, dh_last: Optional[torch.Tensor] = None, *,
                     chunk: int = 0, c: float = 8.0, want_dh0: bool = True,
                     workspace: Optional[Workspace] = None):
    """Backward of rglru_fwd_varlen. Returns (dx, dgate_x, dgate_a, dlambda, dh0 [n, W] or None)."""
    lib = _lib.load()
    dev, T, W, io, n = _varlen_common(x, gate_x, gate_a, lam, cu_seqlens, reset, h0)
    shape = make_shape(1, T, W, io, chunk, c)
    _need(dh, "dh", (T, W), io, dev)
    _opt(dh_last, "dh_last", (n, W), torch.float32, dev)
    _need(ckpt, "ckpt", (rglru_ckpt_elems(shape),), torch.float32, dev)
    dx = torch.empty_like(x)
    dgate_x = torch.empty_like(x)
    dgate_a = torch.empty_like(x)
    dlam = torch.empty((W,), dtype=torch.float32, device=dev)
    dh0 = torch.empty((n, W), dtype=torch.float32, device=dev) if want_dh0 else None
    ws = workspace if workspace is not None else default_workspace(dev)
    buf = ws.get(rglru_varlen_workspace_bytes(shape, n))
    st = lib.rglru_bwd_varlen(ctypes.byref(shape), _ptr(cu_seqlens), n, _ptr(x), _ptr(gate_x), _ptr(gate_a),
                              _ptr(lam), _ptr(reset), _ptr(h0), _ptr(ckpt), _ptr(dh), _ptr(dh_last), _ptr(dx),
                              _ptr(dgate_x), _ptr(dgate_a), _ptr(dlam), _ptr(dh0), _ptr(buf), buf.numel(),
                              _stream(dev))
    _lib.check(st, "rglru_bwd_varlen")
    return dx, dgate_x, dgate_a, dlam, dh0


def rglru_blockdiag_gate_proj_fwd(x: torch.Tensor, w_x: torch.Tensor, b_x: Optional[torch.Tensor],
                                  w_a: torch.Tensor, b_a: Optional[torch.Tensor], *,
                                  gate_x: Optional[torch.Tensor] = None, gate_a: Optional[torch.Tensor] = None):
    """Both block-diagonal gate projections of x [T, W] (bf16). Returns (gate_x, gate_a)."""
    lib = _lib.load()
    dev = x.device
    T, W = x.shape
    nb, bs, _ = w_x.shape
    _need(x, "x", (T, W), torch.bfloat16, dev)
    _need(w_x, "w_x", (nb, bs, bs), torch.bfloat16, dev)
    _need(w_a, "w_a", (nb, bs, bs), torch.bfloat16, dev)
    _opt(b_x, "b_x", (W,), torch.bfloat16, dev)
    _opt(b_a, "b_a", (W,), torch.bfloat16, dev)
    gate_x = torch.empty_like(x) if gate_x is None else _need(gate_x, "gate_x", (T, W), torch.bfloat16, dev)
    gate_a = torch.empty_like(x) if gate_a is None else _need(gate_a, "gate_a", (T, W), torch.bfloat16, dev)
    st = lib.rglru_blockdiag_gate_proj_fwd(T, W, bs, _ptr(x), _ptr(w_x), _ptr(b_x), _ptr(w_a), _ptr(b_a),
                                           _ptr(gate_x), _ptr(gate_a), _stream(dev))
    _lib.check(st, "rglru_blockdiag_gate_proj_fwd")
    return gate_x, gate_a


def rglru_blockdiag_fused_fwd(x: torch.Tensor, w_x: torch.Tensor, b_x: Optional[torch.Tensor], w_a: torch.Tensor,
                              b_a: Optional[torch.Tensor], lam: torch.Tensor, reset: Optional[torch.Tensor] = None,
                              h0: Optional[torch.Tensor] = None, *, c: float = 8.0, training: bool = True,
                              want_h_last: bool = True, want_gates: bool = False,
                              h: Optional[torch.Tensor] = None, h_last: Optional[torch.Tensor] = None,
                              ckpt: Optional[torch.Tensor] = None, gate_x: Optional[torch.Tensor] = None,
                              gate_a: Optional[torch.Tensor] = None, workspace: Optional[Workspace] = None):
    """Both gate projections and the forward scan in one call (x [B, L, W] bf16, W a multiple of 256).
    Returns (h, h_last or None, ckpt or None, gate_x or None, gate_a or None)."""
    lib = _lib.load()
    dev = x.device
    B, L, W = x.shape
    nb = W // 256
    _need(x, "x", (B, L, W), torch.bfloat16, dev)
    _need(w_x, "w_x", (nb, 256, 256), torch.bfloat16, dev)
    _need(w_a, "w_a", (nb, 256, 256), torch.bfloat16, dev)
    _opt(b_x, "b_x", (W,), torch.bfloat16, dev)
    _opt(b_a, "b_a", (W,), torch.bfloat16, dev)
    _need(lam, "lambda", (W,), torch.float32, dev)
    _opt(reset, "reset", (B, L), torch.uint8, dev)
    _opt(h0, "h0", (B, W), torch.float32, dev)
    shape = make_shape(B, L, W, torch.bfloat16, 0, c)
    if h is None:
        h = torch.empty((B, L, W), dtype=torch.bfloat16, device=dev)
    _need(h, "h", (B, L, W), torch.bfloat16, dev)
    if h_last is None and want_h_last:
        h_last = torch.empty((B, W), dtype=torch.float32, device=dev)
    _opt(h_last, "h_last", (B, W), torch.float32, dev)
    if ckpt is None and training:
        ckpt = torch.empty(rglru_ckpt_elems(shape), dtype=torch.float32, device=dev)
    if ckpt is not None:
        _need(ckpt, "ckpt", (rglru_ckpt_elems(shape),), torch.float32, dev)
    if want_gates:
        gate_x = torch.empty_like(x) if gate_x is None else gate_x
        gate_a = torch.empty_like(x) if gate_a is None else gate_a
    _opt(gate_x, "gate_x", (B, L, W), torch.bfloat16, dev)
    _opt(gate_a, "gate_a", (B, L, W), torch.bfloat16, dev)
    ws = workspace if workspace is not None else default_workspace(dev)
    nbytes = int(lib.rglru_blockdiag_fused_fwd_workspace_bytes(ctypes.byref(shape)))
    buf = ws.get(max(nbytes, rglru_workspace_bytes(shape)))
    st = lib.rglru_blockdiag_fused_fwd(ctypes.byref(shape), _ptr(x), _ptr(w_x), _ptr(b_x), _ptr(w_a), _ptr(b_a),
                                       _ptr(lam), _ptr(reset), _ptr(h0), _ptr(h), _ptr(h_last), _ptr(ckpt),
                                       _ptr(gate_x), _ptr(gate_a), _ptr(buf), buf.numel(), _stream(dev))
    _lib.check(st, "rglru_blockdiag_fused_fwd")
    return h, h_last, ckpt, gate_x, gate_a


def rglru_blockdiag_gate_proj_bwd(x: torch.Tensor, w_x: torch.Tensor, w_a: torch.Tensor,
                                  dgate_x: torch.Tensor, dgate_a: torch.Tensor,
                                  dx_in: Optional[torch.Tensor] = None, *, want_db: bool = True,
                                  dx_out: Optional[torch.Tensor] = None):
    """Backward of both projections. Returns (dx, dw_x, db_x, dw_a, db_a)."""
    lib = _lib.load()
    dev = x.device
    T, W = x.shape
    nb, bs, _ = w_x.shape
    for t, n in ((x, "x"), (dgate_x, "dgate_x"), (dgate_a, "dgate_a")):
        _need(t, n, (T, W), torch.bfloat16, dev)
    _need(w_x, "w_x", (nb, bs, bs), torch.bfloat16, dev)
    _need(w_a, "w_a", (nb, bs, bs), torch.bfloat16, dev)
    _opt(dx_in, "dx_in", (T, W), torch.bfloat16, dev)
    dx_out = torch.empty_like(x) if dx_out is None else _need(dx_out, "dx_out", (T, W), torch.bfloat16, dev)
    dw_x = torch.empty((nb, bs, bs), dtype=torch.float32, device=dev)
    dw_a = torch.empty((nb, bs, bs), dtype=torch.float32, device=dev)
    db_x = torch.empty((W,), dtype=torch.float32, device=dev) if want_db else None
    db_a = torch.empty((W,), dtype=torch.float32, device=dev) if want_db else None
    nws = int(lib.rglru_blockdiag_gate_proj_bwd_workspace_bytes(T, W, bs))
    ws = torch.empty(max(nws, 256), dtype=torch.uint8, device=dev)
    st = lib.rglru_blockdiag_gate_proj_bwd(T, W, bs, _ptr(x), _ptr(w_x), _ptr(w_a), _ptr(dgate_x),
                                           _ptr(dgate_a), _ptr(dx_in), _ptr(dx_out), _ptr(dw_x), _ptr(db_x),
                                           _ptr(dw_a), _ptr(db_a), _ptr(ws), ws.numel(), _stream(dev))
    _lib.check(st, "rglru_blockdiag_gate_proj_bwd")
    return dx_out, dw_x, db_x, dw_a, db_a


class _RGLRU(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, gate_x, gate_a, lam, h0, reset, chunk, c):
        h, h_last, ckpt = rglru_fwd(x, gate_x, gate_a, lam, reset, h0, chunk=chunk, c=c, training=True)
        ctx.save_for_backward(x, gate_x, gate_a, lam, reset, ckpt)
        ctx.has_h0 = h0 is not None
        ctx.chunk, ctx.c = chunk, c
        return h, h_last

    @staticmethod
    def backward(ctx, dh, dh_last):
        x, gate_x, gate_a, lam, reset, ckpt = ctx.saved_tensors
        dh = torch.zeros_like(x) if dh is None else dh.contiguous().to(x.dtype)
        dh_last = None if dh_last is None else dh_last.contiguous().float()
        dx, dgx, dga, dlam, dh0 = rglru_bwd(x, gate_x, gate_a, lam, reset, ckpt, dh, dh_last,
                                            chunk=ctx.chunk, c=ctx.c, want_dh0=ctx.has_h0)
        return dx, dgx, dga, dlam, (dh0 if ctx.has_h0 else None), None, None, None


def rglru(x, gate_x, gate_a, lam, h0=None, reset=None, *, chunk: int = 0, c: float = 8.0):
    """Differentiable RG-LRU scan: returns (h, h_last). Gradients flow to x, gate_x, gate_a, lambda and h0."""
    return _RGLRU.apply(x, gate_x, gate_a, lam, h0, reset, chunk, c)


def _delta_common(q, k, v, g, beta, scale, initial_state, cu_seqlens, state_v_first, output_final_state, o,
                  final_state):
    dev = q.device
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, T, H, D]")
    B, T, Hk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    io = q.dtype
    if io not in _IO:
        raise ValueError(f"unsupported dtype {io}")
    _need(q, "q", (B, T, Hk, Dk), io, dev)
    _need(k, "k", (B, T, Hk, Dk), io, dev)
    _need(v, "v", (B, T, Hv, Dv), io, dev)
    kda = g.dim() == 4
    _need(g, "g", (B, T, Hv, Dk) if kda else (B, T, Hv), torch.float32, dev)
    _need(beta, "beta", (B, T, Hv), torch.float32, dev)
    n = B
    if cu_seqlens is not None:
        if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
            raise ValueError("cu_seqlens must be [N + 1]")
        n = cu_seqlens.numel() - 1
        _need(cu_seqlens, "cu_seqlens", (n + 1,), torch.int32, dev)
    sshape = (n, Hv, Dv, Dk) if state_v_first else (n, Hv, Dk, Dv)
    _opt(initial_state, "initial_state", sshape, torch.float32, dev)
    o = torch.empty_like(v) if o is None else _need(o, "o", (B, T, Hv, Dv), io, dev)
    if output_final_state:
        final_state = (torch.empty(sshape, dtype=torch.float32, device=dev) if final_state is None
                       else _need(final_state, "final_state", sshape, torch.float32, dev))
    else:
        final_state = None
    sc = (1.0 / float(Dk) ** 0.5) if scale is None else float(scale)
    shape = _lib.rglru_delta_shape_t(B, T, Hk, Hv, Dk, Dv, _IO[io],
                                     _lib.RGLRU_DELTA_KDA if kda else _lib.RGLRU_DELTA_GDN,
                                     int(bool(state_v_first)), sc)
    return shape, n, o, final_state


def rglru_delta_ckpt_elems(shape: _lib.rglru_delta_shape_t, n_seqs: int = 0) -> int:
    return int(_lib.load().rglru_delta_ckpt_elems(ctypes.byref(shape), int(n_seqs)))


def rglru_delta_rule_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor, *,
                         scale: Optional[float] = None, initial_state: Optional[torch.Tensor] = None,
                         cu_seqlens: Optional[torch.Tensor] = None, state_v_first: bool = False,
                         output_final_state: bool = True, o: Optional[torch.Tensor] = None,
                         final_state: Optional[torch.Tensor] = None, training: bool = False,
                         ckpt: Optional[torch.Tensor] = None):
    """Gated delta rule forward, token recurrence (GDN when g is [B, T, Hv], KDA when [B, T, Hv, Dk]).

    q, k [B, T, Hk, Dk] and v [B, T, Hv, Dv] in bfloat16 or float32 (one dtype);
    g, beta float32; states float32 [N, Hv, Dk, Dv] ([N, Hv, Dv, Dk] with
    state_v_first), N = B, or the number of sequences when cu_seqlens (int32
    [N + 1], B = 1) packs them. scale defaults to 1 / sqrt(Dk).
    With training (or a ckpt tensor given), the forward also writes the
    float32 checkpoint rglru_delta_rule_bwd needs. Returns (o [B, T, Hv, Dv],
    final state or None), plus the checkpoint when training.
    """
    lib = _lib.load()
    shape, n, o, final_state = _delta_common(q, k, v, g, beta, scale, initial_state, cu_seqlens, state_v_first,
                                             output_final_state, o, final_state)
    n_packed = n if cu_seqlens is not None else 0
    if training or ckpt is not None:
        ne = int(lib.rglru_delta_ckpt_elems(ctypes.byref(shape), n_packed))
        ckpt = (torch.empty(max(ne, 1), dtype=torch.float32, device=q.device) if ckpt is None
                else _need(ckpt, "ckpt", (ckpt.numel(),), torch.float32, q.device))
        if ckpt.numel() < ne:
            raise ValueError(f"ckpt needs {ne} elements")
    st = lib.rglru_delta_rule_fwd(ctypes.byref(shape), _ptr(cu_seqlens), n, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                  _ptr(beta), _ptr(initial_state), _ptr(o), _ptr(final_state), _ptr(ckpt),
                                  _stream(q.device))
    _lib.check(st, "rglru_delta_rule_fwd")
    if training or ckpt is not None:
        return o, final_state, ckpt
    return o, final_state


def rglru_delta_bwd_workspace_bytes(shape: _lib.rglru_delta_shape_t, n_seqs: int = 0) -> int:
    """Workspace bytes of rglru_delta_rule_bwd: n_seqs packed sequences, or 0 for B rows."""
    return int(_lib.load().rglru_delta_bwd_workspace_bytes(ctypes.byref(shape), int(n_seqs)))


def rglru_delta_rule_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor,
                         ckpt: torch.Tensor, do: torch.Tensor, dh_last: Optional[torch.Tensor] = None, *,
                         scale: Optional[float] = None, cu_seqlens: Optional[torch.Tensor] = None,
                         state_v_first: bool = False, want_dh0: bool = True, workspace: Optional[torch.Tensor] = None):
    """Backward of rglru_delta_rule_fwd (token form) from its checkpoint.

    Returns (dq, dk, dv, dg, dbeta, dh0): dq, dk, dv in the io dtype, dg and
    dbeta float32 in the shapes of g and beta, dh0 float32 in the layout of the
    states (None unless want_dh0)."""
    lib = _lib.load()
    dev = q.device
    shape, n, _, _ = _delta_common(q, k, v, g, beta, scale, None, cu_seqlens, state_v_first, False, do, None)
    B, T, Hk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    sshape = (n, Hv, Dv, Dk) if state_v_first else (n, Hv, Dk, Dv)
    _opt(dh_last, "dh_last", sshape, torch.float32, dev)
    n_packed = n if cu_seqlens is not None else 0
    ne = int(lib.rglru_delta_ckpt_elems(ctypes.byref(shape), n_packed))
    if not isinstance(ckpt, torch.Tensor) or ckpt.dtype != torch.float32 or ckpt.numel() < ne or ckpt.device != dev:
        raise ValueError(f"ckpt must be a float32 tensor of at least {ne} elements on {dev}")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dg = torch.empty(g.shape, dtype=torch.float32, device=dev)
    dbeta = torch.empty(beta.shape, dtype=torch.float32, device=dev)
    dh0 = torch.empty(sshape, dtype=torch.float32, device=dev) if want_dh0 else None
    nbytes = int(lib.rglru_delta_bwd_workspace_bytes(ctypes.byref(shape), n_packed))
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    st = lib.rglru_delta_rule_bwd(ctypes.byref(shape), _ptr(cu_seqlens), n, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                  _ptr(beta), _ptr(ckpt), _ptr(do), _ptr(dh_last), _ptr(dq), _ptr(dk), _ptr(dv),
                                  _ptr(dg), _ptr(dbeta), _ptr(dh0), _ptr(workspace), workspace.numel(),
                                  _stream(dev))
    _lib.check(st, "rglru_delta_rule_bwd")
    return dq, dk, dv, dg, dbeta, dh0


def rglru_delta_chunk_workspace_bytes(shape: _lib.rglru_delta_shape_t, n_seqs: int = 0) -> int:
    """Workspace bytes of rglru_delta_chunk_fwd: n_seqs packed sequences, or 0 for B rows."""
    return int(_lib.load().rglru_delta_chunk_workspace_bytes(ctypes.byref(shape), int(n_seqs)))


def rglru_delta_chunk_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor, *,
                          scale: Optional[float] = None, initial_state: Optional[torch.Tensor] = None,
                          cu_seqlens: Optional[torch.Tensor] = None, state_v_first: bool = False,
                          output_final_state: bool = True, o: Optional[torch.Tensor] = None,
                          final_state: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """Gated delta rule forward for GDN in chunk form (64-token chunks, bf16 MFMA, float32 state).

    Same arguments and results as rglru_delta_rule_fwd (packed sequences
    included); bf16 q, k, v, Dk 64 or 128, Dv a multiple of 32 up to 256.
    workspace: a uint8 device tensor of at least rglru_delta_chunk_workspace_bytes
    bytes (allocated here when None)."""
    lib = _lib.load()
    if g.dim() != 3:
        raise ValueError("the chunk form takes the GDN decay g [B, T, Hv]")
    shape, n, o, final_state = _delta_common(q, k, v, g, beta, scale, initial_state, cu_seqlens, state_v_first,
                                             output_final_state, o, final_state)
    n_packed = n if cu_seqlens is not None else 0
    nbytes = int(lib.rglru_delta_chunk_workspace_bytes(ctypes.byref(shape), n_packed))
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    st = lib.rglru_delta_chunk_fwd(ctypes.byref(shape), _ptr(cu_seqlens), n_packed, _ptr(q), _ptr(k), _ptr(v),
                                   _ptr(g), _ptr(beta), _ptr(initial_state), _ptr(o), _ptr(final_state),
                                   _ptr(workspace), workspace.numel(), _stream(q.device))
    _lib.check(st, "rglru_delta_chunk_fwd")
    return o, final_state
