"""The C-ABI library without a GPU: it loads, exports every declared entry point,
answers size queries, and rejects bad arguments on the host before any launch."""
import ctypes

import pytest

from gated_linear_recurrence_amd import _lib


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def _shape(B=4, L=2048, W=2048, io=1, chunk=0, c=8.0):
    return _lib.rglru_shape_t(B, L, W, io, chunk, c, 0)


def test_exports_every_declared_symbol(lib):
    names = _lib.header_symbols()
    assert {"rglru_fwd", "rglru_bwd", "rglru_blockdiag_gate_proj_fwd", "rglru_blockdiag_gate_proj_bwd"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.rglru_abi_version() == 1


def test_ckpt_and_workspace_sizes(lib):
    s = _shape()
    assert lib.rglru_ckpt_elems(ctypes.byref(s)) == 4 * 256 * 2048
    s2 = _shape(L=2049)
    assert lib.rglru_ckpt_elems(ctypes.byref(s2)) == 4 * 257 * 2048
    f = lib.rglru_fwd_workspace_bytes(ctypes.byref(s))
    b = lib.rglru_bwd_workspace_bytes(ctypes.byref(s))
    assert f > 256 and b > 256
    assert lib.rglru_workspace_bytes(ctypes.byref(s)) == max(f, b)
    # bigger shapes never need less
    assert lib.rglru_fwd_workspace_bytes(ctypes.byref(_shape(L=4096))) >= f


@pytest.mark.parametrize("bad", [dict(B=0), dict(L=0), dict(W=0), dict(io=7), dict(chunk=24), dict(chunk=512),
                                 dict(c=float("nan")), dict(c=float("inf"))])
def test_invalid_shapes_rejected(lib, bad):
    kw = dict(B=1, L=16, W=64)
    kw.update(bad)
    s = _shape(**kw)
    assert lib.rglru_ckpt_elems(ctypes.byref(s)) == 0
    assert lib.rglru_workspace_bytes(ctypes.byref(s)) == 0
    st = lib.rglru_fwd(ctypes.byref(s), *([None] * 10), 0, None)
    assert st == 1


def test_reserved_field_must_be_zero(lib):
    s = _shape(B=1, L=16, W=64)
    s.reserved = 1
    assert lib.rglru_workspace_bytes(ctypes.byref(s)) == 0


def test_null_required_pointers_rejected(lib):
    s = _shape(B=1, L=16, W=64)
    fake = ctypes.c_void_p(0x100000)   # never dereferenced: validation fails first
    args = [fake] * 3 + [fake, None, None, fake, None, None, None]
    assert lib.rglru_fwd(ctypes.byref(s), *args, 1 << 20, None) == 1          # NULL workspace
    assert lib.rglru_bwd(ctypes.byref(s), *([None] * 14), 0, None) == 1


def test_status_strings(lib):
    for st in range(6):
        assert lib.rglru_status_string(st).decode().startswith("RGLRU_")
    assert b"UNKNOWN" in lib.rglru_status_string(99)
