"""ctypes view of librglru.so: the C ABI of include/*.h, nothing more.

The library is loaded from this package directory only. If it is missing, every
entry point raises: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
import re
from ctypes import POINTER, c_float, c_int, c_int32, c_int64, c_size_t, c_uint8, c_void_p

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "librglru.so")
INCLUDE_DIR = os.path.join(os.path.dirname(PKG), "include")
HEADER_PATH = os.path.join(INCLUDE_DIR, "rglru.h")

RGLRU_IO_F32 = 0
RGLRU_IO_BF16 = 1
RGLRU_CKPT_STEPS = 8
HEADER_BYTES = 256   # workspace header: u64 call counter, u32 done counter, u32 error bits
RGLRU_SCRATCH_BYTES = 64 << 20   # the static workspace rglru_fwd_scratch uses, per GPU


class rglru_shape_t(ctypes.Structure):
    _fields_ = [
        ("batch", c_int64),
        ("length", c_int64),
        ("width", c_int64),
        ("io_dtype", c_int32),
        ("chunk", c_int32),
        ("c", c_float),
        ("reserved", c_int32),
    ]


RGLRU_DELTA_GDN = 0
RGLRU_DELTA_KDA = 1


class rglru_delta_shape_t(ctypes.Structure):
    _fields_ = [
        ("batch", c_int64),
        ("length", c_int64),
        ("k_heads", c_int32),
        ("v_heads", c_int32),
        ("k_dim", c_int32),
        ("v_dim", c_int32),
        ("io_dtype", c_int32),
        ("decay", c_int32),
        ("state_v_first", c_int32),
        ("scale", c_float),
    ]


_vp = c_void_p
_SIGNATURES = {
    "rglru_ckpt_elems": (c_size_t, [POINTER(rglru_shape_t)]),
    "rglru_fwd_workspace_bytes": (c_size_t, [POINTER(rglru_shape_t)]),
    "rglru_bwd_workspace_bytes": (c_size_t, [POINTER(rglru_shape_t)]),
    "rglru_workspace_bytes": (c_size_t, [POINTER(rglru_shape_t)]),
    "rglru_fwd": (c_int, [POINTER(rglru_shape_t), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                          c_size_t, _vp]),
    "rglru_bwd": (c_int, [POINTER(rglru_shape_t), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                          _vp, _vp, _vp, _vp, c_size_t, _vp]),
    "rglru_blockdiag_gate_proj_fwd": (c_int, [c_int64, c_int64, c_int64, _vp, _vp, _vp, _vp, _vp, _vp,
                                              _vp, _vp]),
    "rglru_blockdiag_gate_proj_bwd_workspace_bytes": (c_size_t, [c_int64, c_int64, c_int64]),
    "rglru_blockdiag_gate_proj_bwd": (c_int, [c_int64, c_int64, c_int64, _vp, _vp, _vp, _vp, _vp, _vp,
                                              _vp, _vp, _vp, _vp, _vp, _vp, c_size_t, _vp]),
    "rglru_fwd_scratch": (c_int, [POINTER(rglru_shape_t), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "rglru_varlen_workspace_bytes": (c_size_t, [POINTER(rglru_shape_t), c_int64]),
    "rglru_blockdiag_fused_fwd_workspace_bytes": (c_size_t, [POINTER(rglru_shape_t)]),
    "rglru_blockdiag_fused_fwd": (c_int, [POINTER(rglru_shape_t)] + [_vp] * 14 + [c_size_t, _vp]),
    "rglru_fwd_varlen": (c_int, [POINTER(rglru_shape_t), _vp, c_int64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                 _vp, _vp, c_size_t, _vp]),
    "rglru_bwd_varlen": (c_int, [POINTER(rglru_shape_t), _vp, c_int64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                 _vp, _vp, _vp, _vp, _vp, _vp, _vp, c_size_t, _vp]),
    "rglru_delta_rule_fwd": (c_int, [POINTER(rglru_delta_shape_t), _vp, c_int64] + [_vp] * 10),
    "rglru_delta_ckpt_elems": (c_size_t, [POINTER(rglru_delta_shape_t), c_int64]),
    "rglru_delta_bwd_workspace_bytes": (c_size_t, [POINTER(rglru_delta_shape_t), c_int64]),
    "rglru_delta_rule_bwd": (c_int, [POINTER(rglru_delta_shape_t), _vp, c_int64] + [_vp] * 15 + [c_size_t, _vp]),
    "rglru_delta_chunk_workspace_bytes": (c_size_t, [POINTER(rglru_delta_shape_t), c_int64]),
    "rglru_delta_chunk_fwd": (c_int, [POINTER(rglru_delta_shape_t), _vp, c_int64] + [_vp] * 9 + [c_size_t, _vp]),
    "rglru_status_string": (ctypes.c_char_p, [c_int]),
    "rglru_abi_version": (c_int, []),
}

_lib = None


def header_symbols() -> list:
    """Names of the functions the headers under include/ declare."""
    text = ""
    for name in sorted(os.listdir(INCLUDE_DIR)):
        if name.endswith(".h"):
            with open(os.path.join(INCLUDE_DIR, name)) as f:
                text += f.read() + "\n"
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rglru_[a-z0-9_]+)\s*\(", text)))


def load(path: str = LIB_PATH):
    """Loads librglru.so (once) and declares every signature."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is not built; run `python -m gated_linear_recurrence_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class RglruError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = load()
        super().__init__(f"{where}: {lib.rglru_status_string(status).decode()}")
        self.status = status


def check(status: int, where: str) -> None:
    if status != 0:
        raise RglruError(status, where)
