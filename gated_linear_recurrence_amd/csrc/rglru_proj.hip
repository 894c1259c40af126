// Block-diagonal gate projections (MFMA) - entry points.
#include <hip/hip_runtime.h>

#include "common.h"

extern "C" {

size_t rglru_blockdiag_gate_proj_bwd_workspace_bytes(int64_t tokens, int64_t width, int64_t block) {
  (void)tokens; (void)width; (void)block;
  return 0;
}

rglru_status_t rglru_blockdiag_gate_proj_fwd(int64_t, int64_t, int64_t, const void*, const void*, const void*,
                                             const void*, const void*, void*, void*, void*) {
  return RGLRU_ERR_UNSUPPORTED;
}

rglru_status_t rglru_blockdiag_gate_proj_bwd(int64_t, int64_t, int64_t, const void*, const void*, const void*,
                                             const void*, const void*, const void*, void*, float*, float*,
                                             float*, float*, void*, size_t, void*) {
  return RGLRU_ERR_UNSUPPORTED;
}

}  // extern "C"
