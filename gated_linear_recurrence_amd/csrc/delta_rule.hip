// Gated delta rule forward (GDN / KDA), token-recurrent form.
//
// The recurrence is the one the linear_attention reference page names
// recurrent_delta_rule_reference: per value head, decay the [Dk, Dv] state
// (one factor per head for GDN, per key row for KDA), read it with k, write
// beta times the error v - S^T k along k, read the result out with q.
//
// Every column j of the state evolves on its own: the decay scales rows, the
// read S^T k and the read-out S^T q are column dot products, and the write
// adds k times a per-column scalar. So a column is the unit of work. One
// column of Dk float32 values lives in the registers of LPC consecutive lanes
// (R rows each, Dk <= LPC * R); the two column dot products per token are
// reduced across those lanes with DPP adds inside a 16-lane row, and every
// lane of the group ends with the sum. A workgroup of 4 waves holds 256 / LPC
// columns of one head, and the grid is sequences x value heads x column
// blocks, mapped so that the column blocks of one head share an XCD (and its
// L2, which then serves that head's q, k and g to all of them).
//
// Per token every lane needs its R rows of k, q (and of the KDA decays), the
// token's beta and decay, and its column of v. The workgroup stages them for
// TC tokens at a time in LDS as float32 (decays already exponentiated),
// double-buffered: the global loads of the next chunk are issued before the
// current chunk's recurrence and written to LDS after it, with one barrier
// per chunk. Outputs go through LDS too and leave as 16-byte stores. TC is
// 16, or 4 for calls whose sequences are all that short (decode steps),
// where the smaller LDS lets more workgroups be resident. In training mode
// the state entering every 8th token is stored to the checkpoint, each
// slot column-major so a lane's R rows leave as 16-byte pieces.

#include <hip/hip_runtime.h>
#include <cmath>

#include "common.h"
#include "delta_rule.h"

namespace rglru {
namespace delta {

constexpr int kThreads = 256;
constexpr int kTC = 16;  // tokens per staged chunk
constexpr int kTCShort = 4;  // the same for calls of at most this many tokens per sequence

struct DeltaArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  const float* h0;
  void* o;
  float* h_last;
  const int32_t* cu;  // NULL: row n holds tokens [n T, (n + 1) T)
  int64_t T;
  int Hk, Hv, Dk, Dv, grp;
  int n_cb;      // column blocks per head
  int n_blocks;  // workgroups in the grid
  int v_first;
  float scale;
  float* ckpt;        // NULL, or the state entering every 8th token (for the backward)
  int64_t ck_slots;   // checkpoint slots per value head
};

// Workgroup id -> logical block such that consecutive logical blocks share an
// XCD (the dispatcher deals workgroups to the 8 XCDs round robin). Bijective
// for any n.
__device__ __forceinline__ int xcd_remap(int id, int n) {
  const int q = n >> 3, r = n & 7, x = id & 7, pos = id >> 3;
  return x < r ? x * (q + 1) + pos : r * (q + 1) + (x - r) * q + pos;
}

template <int CTRL>
__device__ __forceinline__ float dpp_sum_step(float x) {
  // every control used here reads a valid lane, so no "old" value is needed (mov_dpp leaves it undefined)
  return x + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Sum over each group of LPC consecutive lanes (LPC = 8 or 16, groups aligned
// to LPC); every lane of the group receives the sum. quad_perm [1,0,3,2] and
// [2,3,0,1] fold the quads, row_half_mirror pairs lane i with 7 - i (the
// other quad of its 8), row_mirror pairs i with 15 - i (the other 8 of its 16).
template <int LPC>
__device__ __forceinline__ float group_sum(float x) {
  x = dpp_sum_step<0xB1>(x);
  x = dpp_sum_step<0x4E>(x);
  x = dpp_sum_step<0x141>(x);
  if constexpr (LPC == 16) x = dpp_sum_step<0x140>(x);
  return x;
}

// 16-byte granules of io values.
template <bool BF>
struct Io {
  static constexpr int VW = BF ? 8 : 4;  // elements per 16 bytes
  static constexpr int ES = BF ? 2 : 4;
  __device__ static __forceinline__ void to_f32(const uint4& u, float* f) {
    if constexpr (BF) {
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(w[i] << 16);
        f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      }
    } else {
      f[0] = __uint_as_float(u.x);
      f[1] = __uint_as_float(u.y);
      f[2] = __uint_as_float(u.z);
      f[3] = __uint_as_float(u.w);
    }
  }
  __device__ static __forceinline__ uint4 from_f32(const float* f) {
    if constexpr (BF) {
      return make_uint4(f32x2_to_bf16x2(f[0], f[1]), f32x2_to_bf16x2(f[2], f[3]),
                        f32x2_to_bf16x2(f[4], f[5]), f32x2_to_bf16x2(f[6], f[7]));
    } else {
      return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                        __float_as_uint(f[3]));
    }
  }
};

template <int LPC, int R, bool KDA, bool BF, int TC>
__global__ __launch_bounds__(kThreads) void delta_fwd_kernel(DeltaArgs p) {
  using IO = Io<BF>;
  constexpr int VW = IO::VW;
  constexpr int DKP = LPC * R;            // padded key dimension
  constexpr int CW = kThreads / LPC;      // columns per workgroup
  constexpr int KPT = DKP / VW;           // k granules per token
  constexpr int KG = TC * KPT;           // k (and q) granules per chunk
  constexpr int NKG = (KG + kThreads - 1) / kThreads;
  constexpr int GPT = DKP / 4;            // KDA decay granules (float4) per token
  constexpr int GG = KDA ? TC * GPT : 0;
  constexpr int NGG = KDA ? (GG + kThreads - 1) / kThreads : 1;
  constexpr int VPT = CW / VW;            // v / o granules per token
  constexpr int VG = TC * VPT;
  static_assert(VG <= kThreads && DKP % VW == 0 && CW % VW == 0 && R % 4 == 0, "tiling");

  __shared__ __align__(16) float sk[2][TC][DKP];
  __shared__ __align__(16) float sq[2][TC][DKP];
  __shared__ __align__(16) float sg[2][KDA ? TC : 1][KDA ? DKP : 4];
  __shared__ float sgs[2][TC];
  __shared__ float sb[2][TC];
  __shared__ __align__(16) float sv[2][TC][CW];
  __shared__ __align__(16) float so[2][TC][CW];
  __shared__ float sst[DKP][CW + 1];  // the key-first state slice, for coalesced loads and stores
  constexpr int GQ = CW / 4;          // 16-byte column groups of a state row

  const int bid = xcd_remap(blockIdx.x, p.n_blocks);
  const int cb = bid % p.n_cb;
  const int hn = bid / p.n_cb;
  const int h = hn % p.Hv;
  const int n = hn / p.Hv;
  const int kh = h / p.grp;

  int64_t tok0, len;
  if (p.cu != nullptr) {
    int64_t a = p.cu[n], b = p.cu[n + 1];
    a = a < 0 ? 0 : (a > p.T ? p.T : a);
    b = b < a ? a : (b > p.T ? p.T : b);
    tok0 = a;
    len = b - a;
  } else {
    tok0 = (int64_t)n * p.T;
    len = p.T;
  }

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int rb = lane % LPC;
  const int cl = (tid >> 6) * (64 / LPC) + lane / LPC;
  const int col = cb * CW + cl;
  const bool col_ok = col < p.Dv;

  const int64_t st_base = ((int64_t)n * p.Hv + h) * p.Dk * p.Dv;
  auto st_index = [&](int row) -> int64_t {
    return st_base + (p.v_first ? (int64_t)col * p.Dk + row : (int64_t)row * p.Dv + col);
  };

  float s[R];
  if (!p.v_first) {
    // rows of CW contiguous columns, 16 bytes per load, through LDS
    for (int idx = tid; idx < DKP * GQ; idx += kThreads) {
      const int d = idx / GQ, gq = idx % GQ;
      const int c0 = cb * CW + gq * 4;
      float4 v4 = make_float4(0.f, 0.f, 0.f, 0.f);
      if (p.h0 != nullptr && d < p.Dk && c0 < p.Dv)
        v4 = *reinterpret_cast<const float4*>(p.h0 + st_base + (int64_t)d * p.Dv + c0);
      sst[d][gq * 4] = v4.x;
      sst[d][gq * 4 + 1] = v4.y;
      sst[d][gq * 4 + 2] = v4.z;
      sst[d][gq * 4 + 3] = v4.w;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < R; ++i) s[i] = sst[rb * R + i][cl];
  } else {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int row = rb * R + i;
      s[i] = (p.h0 != nullptr && col_ok && row < p.Dk) ? p.h0[st_index(row)] : 0.0f;
    }
  }

  const char* qb = static_cast<const char*>(p.q);
  const char* kb = static_cast<const char*>(p.k);
  const char* vb = static_cast<const char*>(p.v);
  char* ob = static_cast<char*>(p.o);

  uint4 rk[NKG], rq[NKG];
  float4 rg[NGG];
  uint4 rv = make_uint4(0, 0, 0, 0);
  float rbeta = 0.0f, rgs = 0.0f;

  auto load_chunk = [&](int64_t c) {
    const int64_t t0 = c * TC;
#pragma unroll
    for (int j = 0; j < NKG; ++j) {
      const int idx = tid + kThreads * j;
      const int tt = idx / KPT, part = idx % KPT;
      const bool ok = idx < KG && part * VW < p.Dk && t0 + tt < len;
      rk[j] = rq[j] = make_uint4(0, 0, 0, 0);
      if (ok) {
        const int64_t e = ((tok0 + t0 + tt) * p.Hk + kh) * p.Dk + part * VW;
        rk[j] = *reinterpret_cast<const uint4*>(kb + e * IO::ES);
        rq[j] = *reinterpret_cast<const uint4*>(qb + e * IO::ES);
      }
    }
    if constexpr (KDA) {
#pragma unroll
      for (int j = 0; j < NGG; ++j) {
        const int idx = tid + kThreads * j;
        const int tt = idx / GPT, part = idx % GPT;
        const bool ok = idx < GG && part * 4 < p.Dk && t0 + tt < len;
        rg[j] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (ok) rg[j] = *reinterpret_cast<const float4*>(p.g + ((tok0 + t0 + tt) * p.Hv + h) * p.Dk + part * 4);
      }
    }
    {
      const int tt = tid / VPT, part = tid % VPT;
      const int c0 = cb * CW + part * VW;
      rv = make_uint4(0, 0, 0, 0);
      if (tid < VG && c0 < p.Dv && t0 + tt < len)
        rv = *reinterpret_cast<const uint4*>(vb + (((tok0 + t0 + tt) * p.Hv + h) * p.Dv + c0) * IO::ES);
    }
    if (tid < TC) {
      const bool ok = t0 + tid < len;
      const int64_t e = (tok0 + t0 + tid) * p.Hv + h;
      rbeta = ok ? p.beta[e] : 0.0f;
      if constexpr (!KDA) rgs = ok ? p.g[e] : 0.0f;
    }
  };

  auto store_chunk = [&](int b) {
#pragma unroll
    for (int j = 0; j < NKG; ++j) {
      const int idx = tid + kThreads * j;
      if (idx < KG) {
        const int tt = idx / KPT, part = idx % KPT;
        float f[VW];
        IO::to_f32(rk[j], f);
#pragma unroll
        for (int e = 0; e < VW; e += 4)
          *reinterpret_cast<float4*>(&sk[b][tt][part * VW + e]) = make_float4(f[e], f[e + 1], f[e + 2], f[e + 3]);
        IO::to_f32(rq[j], f);
#pragma unroll
        for (int e = 0; e < VW; e += 4)
          *reinterpret_cast<float4*>(&sq[b][tt][part * VW + e]) = make_float4(f[e], f[e + 1], f[e + 2], f[e + 3]);
      }
    }
    if constexpr (KDA) {
#pragma unroll
      for (int j = 0; j < NGG; ++j) {
        const int idx = tid + kThreads * j;
        if (idx < GG) {
          const int tt = idx / GPT, part = idx % GPT;
          *reinterpret_cast<float4*>(&sg[b][tt][part * 4]) =
              make_float4(expf(rg[j].x), expf(rg[j].y), expf(rg[j].z), expf(rg[j].w));
        }
      }
    }
    if (tid < VG) {
      const int tt = tid / VPT, part = tid % VPT;
      float f[VW];
      IO::to_f32(rv, f);
#pragma unroll
      for (int e = 0; e < VW; e += 4)
        *reinterpret_cast<float4*>(&sv[b][tt][part * VW + e]) = make_float4(f[e], f[e + 1], f[e + 2], f[e + 3]);
    }
    if (tid < TC) {
      sb[b][tid] = rbeta;
      if constexpr (!KDA) sgs[b][tid] = expf(rgs);
    }
  };

  auto step = [&](int b, int t) {
    float kk[R], qq[R];
#pragma unroll
    for (int i = 0; i < R; i += 4) {
      const float4 a = *reinterpret_cast<const float4*>(&sk[b][t][rb * R + i]);
      kk[i] = a.x; kk[i + 1] = a.y; kk[i + 2] = a.z; kk[i + 3] = a.w;
    }
    if constexpr (KDA) {
#pragma unroll
      for (int i = 0; i < R; i += 4) {
        const float4 a = *reinterpret_cast<const float4*>(&sg[b][t][rb * R + i]);
        s[i] *= a.x; s[i + 1] *= a.y; s[i + 2] *= a.z; s[i + 3] *= a.w;
      }
    } else {
      const float gam = sgs[b][t];
#pragma unroll
      for (int i = 0; i < R; ++i) s[i] *= gam;
    }
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int i = 0; i < R; i += 2) {
      a0 = fmaf(s[i], kk[i], a0);
      a1 = fmaf(s[i + 1], kk[i + 1], a1);
    }
    const float dk = group_sum<LPC>(a0 + a1);
    const float w = sb[b][t] * (sv[b][t][cl] - dk);
#pragma unroll
    for (int i = 0; i < R; ++i) s[i] = fmaf(w, kk[i], s[i]);
#pragma unroll
    for (int i = 0; i < R; i += 4) {
      const float4 a = *reinterpret_cast<const float4*>(&sq[b][t][rb * R + i]);
      qq[i] = a.x; qq[i + 1] = a.y; qq[i + 2] = a.z; qq[i + 3] = a.w;
    }
    float c0 = 0.f, c1 = 0.f;
#pragma unroll
    for (int i = 0; i < R; i += 2) {
      c0 = fmaf(s[i], qq[i], c0);
      c1 = fmaf(s[i + 1], qq[i + 1], c1);
    }
    const float ov = group_sum<LPC>(c0 + c1);
    if (rb == 0) so[b][t][cl] = p.scale * ov;
  };

  // the state entering the sequence's token 8 j into checkpoint slot j, column-major [Dv][Dk]: a
  // lane's R rows are contiguous, stored 16 bytes at a time (Dk is a multiple of 8, so a group of
  // 4 rows is wholly inside it or wholly past it)
  const int64_t ck_first = (int64_t)h * p.ck_slots + delta_ckpt_base(p.cu != nullptr, p.T, n, tok0);
  auto store_ckpt = [&](int64_t j) {
    if (!col_ok) return;
    float* ck = p.ckpt + (ck_first + j) * p.Dk * p.Dv + (int64_t)col * p.Dk;
#pragma unroll
    for (int i = 0; i < R; i += 4)
      if (rb * R + i < p.Dk)
        *reinterpret_cast<float4*>(ck + rb * R + i) = make_float4(s[i], s[i + 1], s[i + 2], s[i + 3]);
  };
  // chunk c's tokens; in training mode also the state after each of its 8-token intervals but the
  // last (the one entering the chunk is stored before)
  auto compute = [&](int b, int nt, int64_t c) {
    const bool ck = p.ckpt != nullptr;
    if (nt == TC) {
#pragma unroll
      for (int t = 0; t < TC; ++t) {
        step(b, t);
        if ((t + 1) % kDeltaCkpt == 0 && t + 1 < TC && ck) store_ckpt((c * TC + t + 1) / kDeltaCkpt);
      }
    } else {
      for (int t = 0; t < nt; ++t) {
        step(b, t);
        if ((t + 1) % kDeltaCkpt == 0 && t + 1 < nt && ck) store_ckpt((c * TC + t + 1) / kDeltaCkpt);
      }
    }
  };

  auto write_out = [&](int b, int64_t c) {
    const int64_t t0 = c * TC;
    const int tt = tid / VPT, part = tid % VPT;
    const int c0 = cb * CW + part * VW;
    if (tid < VG && c0 < p.Dv && t0 + tt < len) {
      float f[VW];
#pragma unroll
      for (int e = 0; e < VW; ++e) f[e] = so[b][tt][part * VW + e];
      *reinterpret_cast<uint4*>(ob + (((tok0 + t0 + tt) * p.Hv + h) * p.Dv + c0) * IO::ES) = IO::from_f32(f);
    }
  };

  const int64_t nch = (len + TC - 1) / TC;
  if (nch > 0) {
    load_chunk(0);
    store_chunk(0);
    __syncthreads();
    for (int64_t c = 0; c < nch; ++c) {
      const int b = (int)(c & 1);
      if (c + 1 < nch) load_chunk(c + 1);
      if (p.ckpt != nullptr) store_ckpt(c * TC / kDeltaCkpt);
      const int64_t rem = len - c * TC;
      compute(b, rem < TC ? (int)rem : TC, c);
      if (c + 1 < nch) store_chunk(b ^ 1);
      if (c > 0) write_out(b ^ 1, c - 1);
      __syncthreads();
    }
    write_out((int)((nch - 1) & 1), nch - 1);
  }

  if (p.h_last != nullptr && !p.v_first) {
    __syncthreads();  // every lane has read its initial slice
#pragma unroll
    for (int i = 0; i < R; ++i) sst[rb * R + i][cl] = s[i];
    __syncthreads();
    for (int idx = tid; idx < DKP * GQ; idx += kThreads) {
      const int d = idx / GQ, gq = idx % GQ;
      const int c0 = cb * CW + gq * 4;
      if (d < p.Dk && c0 < p.Dv)
        *reinterpret_cast<float4*>(p.h_last + st_base + (int64_t)d * p.Dv + c0) =
            make_float4(sst[d][gq * 4], sst[d][gq * 4 + 1], sst[d][gq * 4 + 2], sst[d][gq * 4 + 3]);
    }
  } else if (p.h_last != nullptr && col_ok) {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int row = rb * R + i;
      if (row < p.Dk) p.h_last[st_index(row)] = s[i];
    }
  }
}

template <int LPC, int R, bool KDA, bool BF, int TC>
hipError_t launch(const DeltaArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((delta_fwd_kernel<LPC, R, KDA, BF, TC>), dim3(a.n_blocks), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

template <int LPC, int R, int TC>
hipError_t launch_dt(const DeltaArgs& a, bool kda, bool bf, hipStream_t st) {
  if (kda) return bf ? launch<LPC, R, true, true, TC>(a, st) : launch<LPC, R, true, false, TC>(a, st);
  return bf ? launch<LPC, R, false, true, TC>(a, st) : launch<LPC, R, false, false, TC>(a, st);
}

// The tiling of a call: lanes per state column (which sets the columns per workgroup and so the
// grid) and the launcher of the matching instantiation, chosen in one place.
struct Tiling {
  int lpc;
  hipError_t (*launch)(const DeltaArgs&, bool, bool, hipStream_t);
};

// Sequences of at most kTCShort tokens (decode steps) stage kTCShort tokens: a quarter of the
// LDS, so more workgroups are resident; for Dk <= 128 their columns also sit on 8 lanes of 16
// rows, so each workgroup moves twice the state per memory round trip. Each sequence is then one
// chunk, whose checkpoint slot is the same under either chunk length.
inline Tiling pick_tiling(int64_t k_dim, bool short_call) {
  if (short_call) {
    if (k_dim <= 64) return {8, launch_dt<8, 8, kTCShort>};
    if (k_dim <= 128) return {8, launch_dt<8, 16, kTCShort>};
    return {16, launch_dt<16, 16, kTCShort>};
  }
  if (k_dim <= 64) return {8, launch_dt<8, 8, kTC>};
  if (k_dim <= 128) return {16, launch_dt<16, 8, kTC>};
  return {16, launch_dt<16, 16, kTC>};
}

}  // namespace delta
}  // namespace rglru

using namespace rglru;

extern "C" size_t rglru_delta_ckpt_elems(const rglru_delta_shape_t* sp, int64_t n_seqs) {
  if (sp == nullptr || sp->batch < 0 || sp->length < 0 || sp->batch > (int64_t(1) << 40) ||
      sp->length > (int64_t(1) << 40) || sp->v_heads < 1 || sp->k_dim < 1 || sp->v_dim < 1 || n_seqs < 0 ||
      (n_seqs > 0 && sp->batch != 1))
    return 0;
  const int64_t slots = delta_ckpt_slots(n_seqs > 0, sp->length, sp->batch, n_seqs);
  return (size_t)slots * sp->v_heads * sp->k_dim * sp->v_dim;
}

extern "C" rglru_status_t rglru_delta_rule_fwd(const rglru_delta_shape_t* sp, const int32_t* cu_seqlens,
                                               int64_t n_seqs, const void* q, const void* k, const void* v,
                                               const float* g, const float* beta, const float* h0, void* o,
                                               float* h_last, float* ckpt, void* stream) {
  if (sp == nullptr) return RGLRU_ERR_INVALID_ARGUMENT;
  const rglru_delta_shape_t s = *sp;
  if (s.batch < 0 || s.length < 0 || s.batch > (int64_t(1) << 40) || s.length > (int64_t(1) << 40) ||
      (s.batch > 0 && s.length >= (int64_t(1) << 40) / s.batch))
    return RGLRU_ERR_INVALID_ARGUMENT;
  if (s.k_heads < 1 || s.v_heads < s.k_heads || s.v_heads >= (1 << 16) || s.v_heads % s.k_heads != 0)
    return RGLRU_ERR_INVALID_ARGUMENT;
  if (s.k_dim < 1 || s.v_dim < 1 || s.k_dim > (1 << 16) || s.v_dim > (1 << 16)) return RGLRU_ERR_INVALID_ARGUMENT;
  if (s.io_dtype != RGLRU_IO_F32 && s.io_dtype != RGLRU_IO_BF16) return RGLRU_ERR_INVALID_ARGUMENT;
  if (s.decay != RGLRU_DELTA_GDN && s.decay != RGLRU_DELTA_KDA) return RGLRU_ERR_INVALID_ARGUMENT;
  if (s.state_v_first != 0 && s.state_v_first != 1) return RGLRU_ERR_INVALID_ARGUMENT;
  if (!std::isfinite(s.scale)) return RGLRU_ERR_INVALID_ARGUMENT;
  int64_t N = s.batch;
  if (cu_seqlens != nullptr) {
    if (s.batch != 1 || n_seqs < 1 || n_seqs >= (int64_t(1) << 30)) return RGLRU_ERR_INVALID_ARGUMENT;
    N = n_seqs;
  }
  const int64_t tokens = s.batch * s.length;
  const bool kda = s.decay == RGLRU_DELTA_KDA;
  if (tokens > 0 && (q == nullptr || k == nullptr || v == nullptr || g == nullptr || beta == nullptr ||
                     o == nullptr))
    return RGLRU_ERR_INVALID_ARGUMENT;
  const delta::Tiling tl = delta::pick_tiling(s.k_dim, s.length <= delta::kTCShort);
  const int cw = delta::kThreads / tl.lpc;
  const int64_t n_cb = ceil_div(s.v_dim, cw);
  const int64_t blocks = N * s.v_heads * n_cb;
  if (blocks >= (int64_t(1) << 31)) return RGLRU_ERR_INVALID_ARGUMENT;
  if (s.k_dim > 256 || s.k_dim % 8 != 0 || s.v_dim % 8 != 0) return RGLRU_ERR_UNSUPPORTED;
  if (!aligned_to(q, 16) || !aligned_to(k, 16) || !aligned_to(v, 16) || !aligned_to(o, 16) ||
      !aligned_to(g, kda ? 16 : 4) || !aligned_to(beta, 4) || !aligned_to(h0, 16) || !aligned_to(h_last, 16) || !aligned_to(ckpt, 16) ||
      !aligned_to(cu_seqlens, 4))
    return RGLRU_ERR_MISALIGNED;
  if (blocks == 0 || (tokens == 0 && h_last == nullptr)) return RGLRU_OK;

  delta::DeltaArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.beta = beta;
  a.h0 = h0;
  a.o = o;
  a.h_last = h_last;
  a.cu = cu_seqlens;
  a.T = s.length;
  a.Hk = s.k_heads;
  a.Hv = s.v_heads;
  a.Dk = s.k_dim;
  a.Dv = s.v_dim;
  a.grp = s.v_heads / s.k_heads;
  a.n_cb = (int)n_cb;
  a.n_blocks = (int)blocks;
  a.v_first = s.state_v_first;
  a.scale = s.scale;
  a.ckpt = ckpt;
  a.ck_slots = delta_ckpt_slots(cu_seqlens != nullptr, s.length, s.batch, n_seqs);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool bf = s.io_dtype == RGLRU_IO_BF16;
  const hipError_t e = tl.launch(a, kda, bf, st);
  return e == hipSuccess ? RGLRU_OK : RGLRU_ERR_HIP;
}
