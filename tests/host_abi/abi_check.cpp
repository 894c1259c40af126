// Host-side checks of the C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer around the library's host code (host-only
// compile: no kernel runs). Exercises every size query, the status strings
// and the argument-validation paths of every entry point, which must return
// an error code without touching the GPU. Prints one line per failed
// expectation and exits nonzero if any failed.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>

#include "delta_rule.h"
#include "rglru.h"

extern "C" const char* host_abi_status_of_int(int v);

static int g_fail = 0;

#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      std::printf("FAIL line %d: %s\n", __LINE__, #cond);              \
      ++g_fail;                                                        \
    }                                                                  \
  } while (0)

static rglru_shape_t shape(int64_t b, int64_t l, int64_t w, int32_t io, int32_t chunk = 0, float c = 8.0f) {
  rglru_shape_t s;
  std::memset(&s, 0, sizeof(s));
  s.batch = b;
  s.length = l;
  s.width = w;
  s.io_dtype = io;
  s.chunk = chunk;
  s.c = c;
  s.reserved = 0;
  return s;
}

int main() {
  EXPECT(rglru_abi_version() == RGLRU_ABI_VERSION);
  // any int a C caller may pass (through a C translation unit: in C++ an
  // enum value outside the enumerators' range is itself undefined)
  for (int st = -1; st <= 8; ++st) {
    const char* m = host_abi_status_of_int(st);
    EXPECT(m != nullptr && std::strlen(m) > 0);
  }

  // size queries on valid shapes: nonzero, and the combined workspace covers both directions
  const int64_t sizes[][3] = {{1, 1, 1}, {1, 64, 64}, {4, 2048, 2048}, {3, 777, 300}, {1, 32805, 4096}, {8, 4096, 2560}};
  for (auto& z : sizes) {
    for (int io : {0, 1}) {
      for (int chunk : {0, 8, 16, 32, 64, 128, 256}) {
        rglru_shape_t s = shape(z[0], z[1], z[2], io, chunk);
        const size_t ck = rglru_ckpt_elems(&s);
        const size_t f = rglru_fwd_workspace_bytes(&s);
        const size_t b = rglru_bwd_workspace_bytes(&s);
        const size_t a = rglru_workspace_bytes(&s);
        EXPECT(ck == static_cast<size_t>(z[0] * ((z[1] + RGLRU_CKPT_STEPS - 1) / RGLRU_CKPT_STEPS) * z[2]));
        EXPECT(f > 0 && b > 0 && a >= f && a >= b);
        if (z[0] == 1) EXPECT(rglru_varlen_workspace_bytes(&s, 3) >= f);
        const size_t fz = rglru_blockdiag_fused_fwd_workspace_bytes(&s);
        EXPECT((io == 1 && z[2] % 256 == 0) ? fz > f : fz == 0);
      }
    }
  }
  EXPECT(rglru_blockdiag_gate_proj_bwd_workspace_bytes(8192, 2048, 256) > 0);
  EXPECT(rglru_blockdiag_gate_proj_bwd_workspace_bytes(1, 256, 256) > 0);

  // invalid shapes: every query returns 0, every entry point INVALID_ARGUMENT
  const int64_t big = std::numeric_limits<int64_t>::max();
  rglru_shape_t bad[] = {
      shape(0, 64, 64, 1),        shape(1, 0, 64, 1),         shape(1, 64, 0, 1),
      shape(-1, 64, 64, 1),       shape(1, -5, 64, 1),        shape(1, 64, -64, 1),
      shape(1, 64, 64, 7),        shape(1, 64, 64, 1, 24),    shape(1, 64, 64, 1, 512),
      shape(big, 64, 64, 1),      shape(1, big, 64, 1),       shape(1, 64, big, 1),
      shape(big, big, big, 1),    shape(1 << 25, 64, 64, 1),  shape(1, 64, 64, 1, 0, std::numeric_limits<float>::quiet_NaN()),
      shape(1, 64, 64, 1, 0, std::numeric_limits<float>::infinity()),
  };
  bad[0].reserved = 0;
  rglru_shape_t res = shape(1, 64, 64, 1);
  res.reserved = 1;
  alignas(256) static unsigned char buf[1 << 16];
  void* p = buf;
  auto check_bad = [&](const rglru_shape_t& s) {
    EXPECT(rglru_ckpt_elems(&s) == 0);
    EXPECT(rglru_fwd_workspace_bytes(&s) == 0);
    EXPECT(rglru_bwd_workspace_bytes(&s) == 0);
    EXPECT(rglru_workspace_bytes(&s) == 0);
    EXPECT(rglru_varlen_workspace_bytes(&s, 1) == 0);
    EXPECT(rglru_blockdiag_fused_fwd_workspace_bytes(&s) == 0);
    EXPECT(rglru_fwd(&s, p, p, p, (const float*)p, nullptr, nullptr, p, nullptr, nullptr, p, sizeof(buf), nullptr) ==
           RGLRU_ERR_INVALID_ARGUMENT);
    EXPECT(rglru_bwd(&s, p, p, p, (const float*)p, nullptr, (const float*)p, p, nullptr, p, p, p, (float*)p, nullptr,
                     p, sizeof(buf), nullptr) == RGLRU_ERR_INVALID_ARGUMENT);
    EXPECT(rglru_fwd_scratch(&s, p, p, p, (const float*)p, nullptr, nullptr, p, nullptr, nullptr, nullptr) ==
           RGLRU_ERR_INVALID_ARGUMENT);
    EXPECT(rglru_blockdiag_fused_fwd(&s, p, p, nullptr, p, nullptr, (const float*)p, nullptr, nullptr, p, nullptr,
                                     nullptr, nullptr, nullptr, p, sizeof(buf), nullptr) == RGLRU_ERR_INVALID_ARGUMENT);
  };
  for (auto& s : bad) check_bad(s);
  check_bad(res);
  EXPECT(rglru_ckpt_elems(nullptr) == 0);
  EXPECT(rglru_workspace_bytes(nullptr) == 0);
  EXPECT(rglru_fwd(nullptr, p, p, p, (const float*)p, nullptr, nullptr, p, nullptr, nullptr, p, sizeof(buf), nullptr) ==
         RGLRU_ERR_INVALID_ARGUMENT);

  // valid shape, bad pointers: NULL required pointers, misalignment, workspace too small
  rglru_shape_t s = shape(2, 100, 96, 1);
  const float* fp = (const float*)p;
  EXPECT(rglru_fwd(&s, nullptr, p, p, fp, nullptr, nullptr, p, nullptr, nullptr, p, sizeof(buf), nullptr) ==
         RGLRU_ERR_INVALID_ARGUMENT);
  EXPECT(rglru_fwd(&s, p, p, p, fp, nullptr, nullptr, p, nullptr, nullptr, nullptr, sizeof(buf), nullptr) ==
         RGLRU_ERR_INVALID_ARGUMENT);
  EXPECT(rglru_fwd(&s, buf + 1, p, p, fp, nullptr, nullptr, p, nullptr, nullptr, p, sizeof(buf), nullptr) ==
         RGLRU_ERR_MISALIGNED);
  EXPECT(rglru_fwd(&s, p, p, p, (const float*)(buf + 2), nullptr, nullptr, p, nullptr, nullptr, p, sizeof(buf),
                   nullptr) == RGLRU_ERR_MISALIGNED);
  EXPECT(rglru_fwd(&s, p, p, p, fp, nullptr, nullptr, p, nullptr, nullptr, buf + 16, sizeof(buf), nullptr) ==
         RGLRU_ERR_MISALIGNED);
  EXPECT(rglru_fwd(&s, p, p, p, fp, nullptr, nullptr, p, nullptr, nullptr, p, 16, nullptr) ==
         RGLRU_ERR_WORKSPACE_TOO_SMALL);
  EXPECT(rglru_bwd(&s, p, p, p, fp, nullptr, nullptr, p, nullptr, p, p, p, (float*)p, nullptr, p, sizeof(buf),
                   nullptr) == RGLRU_ERR_INVALID_ARGUMENT);
  EXPECT(rglru_bwd(&s, p, p, p, fp, nullptr, fp, p, nullptr, p, p, p, (float*)p, nullptr, p, 16, nullptr) ==
         RGLRU_ERR_WORKSPACE_TOO_SMALL);

  // packed sequences: batch must be 1, n_seqs in range
  rglru_shape_t sv = shape(1, 500, 64, 1);
  const int32_t* cu = (const int32_t*)p;
  EXPECT(rglru_varlen_workspace_bytes(&sv, 0) == 0);
  EXPECT(rglru_varlen_workspace_bytes(&sv, -3) == 0);
  EXPECT(rglru_varlen_workspace_bytes(&sv, big) == 0);
  rglru_shape_t sv2 = shape(2, 500, 64, 1);
  EXPECT(rglru_varlen_workspace_bytes(&sv2, 3) == 0);
  EXPECT(rglru_fwd_varlen(&sv, cu, 0, p, p, p, fp, nullptr, nullptr, p, nullptr, nullptr, p, sizeof(buf), nullptr) !=
         RGLRU_OK);
  EXPECT(rglru_fwd_varlen(&sv2, cu, 3, p, p, p, fp, nullptr, nullptr, p, nullptr, nullptr, p, sizeof(buf), nullptr) !=
         RGLRU_OK);
  EXPECT(rglru_fwd_varlen(&sv, nullptr, 3, p, p, p, fp, nullptr, nullptr, p, nullptr, nullptr, p, sizeof(buf),
                          nullptr) != RGLRU_OK);
  EXPECT(rglru_bwd_varlen(&sv, cu, 3, nullptr, p, p, fp, nullptr, nullptr, fp, p, nullptr, p, p, p, (float*)p, nullptr,
                          p, sizeof(buf), nullptr) == RGLRU_ERR_INVALID_ARGUMENT);

  // projections: block must be 256, width a multiple of it, sizes in range
  EXPECT(rglru_blockdiag_gate_proj_fwd(0, 256, 256, p, p, nullptr, p, nullptr, p, p, nullptr) ==
         RGLRU_ERR_INVALID_ARGUMENT);
  EXPECT(rglru_blockdiag_gate_proj_fwd(16, 300, 256, p, p, nullptr, p, nullptr, p, p, nullptr) ==
         RGLRU_ERR_INVALID_ARGUMENT);
  EXPECT(rglru_blockdiag_gate_proj_fwd(16, 256, 128, p, p, nullptr, p, nullptr, p, p, nullptr) ==
         RGLRU_ERR_UNSUPPORTED);
  EXPECT(rglru_blockdiag_gate_proj_fwd(16, 256, 256, nullptr, p, nullptr, p, nullptr, p, p, nullptr) ==
         RGLRU_ERR_INVALID_ARGUMENT);
  EXPECT(rglru_blockdiag_gate_proj_fwd(16, 256, 256, buf + 8, p, nullptr, p, nullptr, p, p, nullptr) ==
         RGLRU_ERR_MISALIGNED);
  EXPECT(rglru_blockdiag_gate_proj_fwd(big, 256, 256, p, p, nullptr, p, nullptr, p, p, nullptr) ==
         RGLRU_ERR_INVALID_ARGUMENT);
  EXPECT(rglru_blockdiag_gate_proj_bwd_workspace_bytes(16, 300, 256) == 0);
  EXPECT(rglru_blockdiag_gate_proj_bwd_workspace_bytes(-1, 256, 256) == 0);
  EXPECT(rglru_blockdiag_gate_proj_bwd(16, 256, 256, p, p, p, p, p, nullptr, p, (float*)p, nullptr, (float*)p, nullptr,
                                       p, 16, nullptr) == RGLRU_ERR_WORKSPACE_TOO_SMALL);
  EXPECT(rglru_blockdiag_gate_proj_bwd(16, 256, 256, p, p, p, nullptr, p, nullptr, p, (float*)p, nullptr, (float*)p,
                                       nullptr, p, sizeof(buf), nullptr) == RGLRU_ERR_INVALID_ARGUMENT);

  // fused forward: bf16 only, width a multiple of 256, chunk 0 or 64
  rglru_shape_t sf = shape(2, 100, 512, 1, 32);
  EXPECT(rglru_blockdiag_fused_fwd(&sf, p, p, nullptr, p, nullptr, fp, nullptr, nullptr, p, nullptr, nullptr, nullptr,
                                   nullptr, p, sizeof(buf), nullptr) == RGLRU_ERR_UNSUPPORTED);
  rglru_shape_t sf2 = shape(2, 100, 384, 1);
  EXPECT(rglru_blockdiag_fused_fwd(&sf2, p, p, nullptr, p, nullptr, fp, nullptr, nullptr, p, nullptr, nullptr, nullptr,
                                   nullptr, p, sizeof(buf), nullptr) == RGLRU_ERR_UNSUPPORTED);
  rglru_shape_t sf3 = shape(2, 100, 512, 1);
  EXPECT(rglru_blockdiag_fused_fwd(&sf3, p, p, nullptr, p, nullptr, fp, nullptr, nullptr, p, nullptr, nullptr, nullptr,
                                   nullptr, p, 16, nullptr) == RGLRU_ERR_WORKSPACE_TOO_SMALL);

  // gated delta rule, token and chunk forms: validation paths only (nothing is launched)
  auto dshape = [](int64_t b, int64_t t, int hk, int hv, int dk, int dv, int io, int decay) {
    rglru_delta_shape_t d;
    std::memset(&d, 0, sizeof(d));
    d.batch = b;
    d.length = t;
    d.k_heads = hk;
    d.v_heads = hv;
    d.k_dim = dk;
    d.v_dim = dv;
    d.io_dtype = io;
    d.decay = decay;
    d.state_v_first = 0;
    d.scale = 0.125f;
    return d;
  };
  float* wf = (float*)p;
  const int32_t* dcu = (const int32_t*)p;
  auto dfwd = [&](const rglru_delta_shape_t& d, const void* q, const int32_t* c = nullptr, int64_t n = 0) {
    return rglru_delta_rule_fwd(&d, c, n, q, p, p, fp, fp, nullptr, p, nullptr, nullptr, nullptr);
  };
  rglru_delta_shape_t d = dshape(2, 64, 2, 3, 64, 64, 1, 0);
  EXPECT(dfwd(d, p) == RGLRU_ERR_INVALID_ARGUMENT);  // Hv not a multiple of Hk
  d = dshape(2, 64, 1, 1, 264, 64, 1, 0);
  EXPECT(dfwd(d, p) == RGLRU_ERR_UNSUPPORTED);       // Dk > 256
  d = dshape(2, 64, 1, 1, 64, 12, 1, 1);
  EXPECT(dfwd(d, p) == RGLRU_ERR_UNSUPPORTED);       // Dv not a multiple of 8
  d = dshape(2, 64, 1, 1, 64, 64, 1, 0);
  EXPECT(dfwd(d, buf + 8) == RGLRU_ERR_MISALIGNED);
  EXPECT(dfwd(d, nullptr) == RGLRU_ERR_INVALID_ARGUMENT);
  EXPECT(dfwd(d, p, dcu, 3) == RGLRU_ERR_INVALID_ARGUMENT);  // packed sequences need B = 1
  d.scale = std::numeric_limits<float>::quiet_NaN();
  EXPECT(dfwd(d, p) == RGLRU_ERR_INVALID_ARGUMENT);
  d = dshape(2, 64, 1, 1, 64, 64, 1, 2);
  EXPECT(dfwd(d, p) == RGLRU_ERR_INVALID_ARGUMENT);  // decay kind
  d = dshape(2, 64, 1, 1, 64, 64, 7, 0);
  EXPECT(dfwd(d, p) == RGLRU_ERR_INVALID_ARGUMENT);  // io dtype
  d = dshape(int64_t(1) << 30, int64_t(1) << 11, 1, 1, 64, 64, 1, 0);
  EXPECT(dfwd(d, p) == RGLRU_ERR_INVALID_ARGUMENT);  // 2^41 tokens
  d = dshape(1, 64, 1, 1, 64, 64, 1, 0);
  EXPECT(dfwd(d, p, dcu, 0) == RGLRU_ERR_INVALID_ARGUMENT);  // no sequences
  EXPECT(rglru_delta_rule_fwd(nullptr, nullptr, 0, p, p, p, fp, fp, nullptr, p, nullptr, nullptr, nullptr) ==
         RGLRU_ERR_INVALID_ARGUMENT);
  // checkpoint and backward
  rglru_delta_shape_t b1 = dshape(2, 100, 1, 2, 128, 64, 1, 0);
  EXPECT(rglru_delta_ckpt_elems(&b1, 0) == (size_t)2 * 13 * 2 * 128 * 64);  // ceil(100 / 8) slots a row
  rglru_delta_shape_t b2 = dshape(1, 100, 1, 2, 128, 64, 1, 0);
  EXPECT(rglru_delta_ckpt_elems(&b2, 3) == (size_t)(13 + 3) * 2 * 128 * 64);
  EXPECT(rglru_delta_ckpt_elems(&b1, 3) == 0);   // packed sequences need B = 1
  const size_t bws = rglru_delta_bwd_workspace_bytes(&b1, 0);
  EXPECT(bws > 0 && bws % 256 == 0);
  auto bwd = [&](const rglru_delta_shape_t& d, size_t bytes, const void* dq) {
    return rglru_delta_rule_bwd(&d, nullptr, 0, p, p, p, fp, fp, fp, p, nullptr, (void*)dq, p, p, wf, wf, nullptr, p,
                                bytes, nullptr);
  };
  EXPECT(bwd(b1, 16, p) == RGLRU_ERR_WORKSPACE_TOO_SMALL);
  EXPECT(bwd(b1, bws, nullptr) == RGLRU_ERR_INVALID_ARGUMENT);
  rglru_delta_shape_t b3 = dshape(2, 100, 1, 2, 256, 64, 1, 0);
  EXPECT(bwd(b3, bws, p) == RGLRU_ERR_UNSUPPORTED);   // the backward holds Dk <= 128
  EXPECT(rglru_delta_bwd_workspace_bytes(&b3, 0) == 0);
  rglru_delta_shape_t c1 = dshape(2, 100, 1, 2, 128, 128, 1, 0);
  const size_t cws = rglru_delta_chunk_workspace_bytes(&c1, 0);
  EXPECT(cws > 0 && cws % 256 == 0);
  auto cfwd = [&](const rglru_delta_shape_t& c, size_t bytes, const int32_t* cu = nullptr, int64_t n = 0) {
    return rglru_delta_chunk_fwd(&c, cu, n, p, p, p, fp, fp, nullptr, p, wf, p, bytes, nullptr);
  };
  EXPECT(cfwd(c1, 16) == RGLRU_ERR_WORKSPACE_TOO_SMALL);
  EXPECT(cfwd(c1, cws, dcu, 3) == RGLRU_ERR_INVALID_ARGUMENT);  // packed sequences need B = 1
  rglru_delta_shape_t c2 = dshape(1, 100, 1, 2, 128, 128, 1, 0);
  const size_t pws = rglru_delta_chunk_workspace_bytes(&c2, 5);
  EXPECT(pws > rglru_delta_chunk_workspace_bytes(&c2, 0));  // room for the extra partial chunks and the map
  EXPECT(cfwd(c2, pws, dcu, 0) == RGLRU_ERR_INVALID_ARGUMENT);
  EXPECT(cfwd(c2, pws - 256, dcu, 5) == RGLRU_ERR_WORKSPACE_TOO_SMALL);
  EXPECT(rglru_delta_chunk_workspace_bytes(&c1, 3) == 0);
  const rglru_delta_shape_t unsupported[] = {dshape(2, 100, 1, 2, 128, 128, 1, 1), dshape(2, 100, 1, 2, 96, 128, 1, 0),
                                            dshape(2, 100, 1, 2, 128, 48, 1, 0), dshape(2, 100, 1, 2, 128, 288, 1, 0),
                                            dshape(2, 100, 1, 2, 128, 128, 0, 0)};
  for (const rglru_delta_shape_t& c : unsupported) {
    EXPECT(rglru_delta_chunk_workspace_bytes(&c, 0) == 0);
    EXPECT(cfwd(c, cws) == RGLRU_ERR_UNSUPPORTED);
  }
  EXPECT(rglru_delta_chunk_workspace_bytes(nullptr, 0) == 0);

  std::printf(g_fail ? "host ABI checks: %d failed\n" : "host ABI checks: all passed\n", g_fail);
  return g_fail ? 1 : 0;
}
