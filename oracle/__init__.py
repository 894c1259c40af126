"""Float64 CPU oracles: the RG-LRU scan and its block-diagonal gate projection,
and the gated delta rule (GDN/KDA).

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg. The HIP library and its binding never import,
call or link anything here.
"""
from .delta import chunk_gdn, recurrent_delta_rule, recurrent_delta_rule_backward  # noqa: F401
from .rglru import (  # noqa: F401
    C_DEFAULT,
    blockdiag_proj_backward,
    blockdiag_proj_forward,
    gates,
    rglru_backward,
    rglru_backward_varlen,
    rglru_forward,
    rglru_forward_chunked,
    rglru_forward_varlen,
    sigmoid,
    softplus,
)
