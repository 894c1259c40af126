"""MI355X (gfx950) RG-LRU and gated delta rule: HIP kernels behind a C ABI (include/*.h) and this thin binding."""
from . import _lib
from ._lib import RglruError, header_symbols  # noqa: F401
from .ops import (  # noqa: F401
    Workspace,
    WorkspaceError,
    check_errors,
    make_shape,
    rglru,
    rglru_blockdiag_fused_fwd,
    rglru_blockdiag_gate_proj_bwd,
    rglru_blockdiag_gate_proj_fwd,
    rglru_bwd,
    rglru_bwd_workspace_bytes,
    rglru_delta_bwd_workspace_bytes,
    rglru_delta_chunk_fwd,
    rglru_delta_chunk_workspace_bytes,
    rglru_delta_ckpt_elems,
    rglru_delta_rule_bwd,
    rglru_delta_rule_fwd,
    rglru_ckpt_elems,
    rglru_fwd,
    rglru_fwd_scratch,
    rglru_fwd_varlen,
    rglru_bwd_varlen,
    rglru_varlen_workspace_bytes,
    rglru_fwd_workspace_bytes,
    rglru_workspace_bytes,
)


def load_library():
    """Loads the in-tree librglru.so; raises if it is not built."""
    return _lib.load()
