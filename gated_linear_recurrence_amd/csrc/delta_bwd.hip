// Gated delta rule backward (GDN / KDA), token-recurrent form.
//
// The reverse-mode steps of the token recurrence (the linear_attention
// reference page's recurrent oracle keeps gradients through every input and
// the initial state). With S~ = D S_prev the decayed state, e = v - S~^T k,
// u = beta e, S = S~ + k u^T, o = scale S^T q, and G the gradient of S, each
// token taken in reverse does
//
//   G += scale q do^T;   dq = scale S do;   du = G^T k;   dv = beta du;
//   dbeta = e . du;      dk = G u - beta S~ du;   G~ = G - beta k du^T;
//   dg = <G~, S~> (GDN) or the row sums of G~ * S~ (KDA);   G <- D G~.
//
// Like the forward, a column of the [Dk, Dv] state (and of G) lives in LPC
// lanes, R rows each, and the columns are independent, so each workgroup
// walks its 512 / LPC columns of one head through the tokens in reverse,
// 16-token chunk by chunk: it takes the states entering the chunk and its 9th token from the
// forward's checkpoint (column-major slots, so a lane's rows are contiguous),
// recomputes the chunk's decayed states S~ forward one half chunk at a time,
// each from its own checkpoint (the forward stores one every 8 tokens),
// then runs the reverse steps; the next chunk's inputs are loaded into
// registers after the last reverse step, so they arrive while this chunk's
// sums are flushed. dv and the initial state's gradient belong to single
// columns; dq, dk, dbeta and dg sum over all columns of a head, so the
// workgroup sums its columns in a fixed order (DPP adds and permlane swaps
// inside a wave, then the waves' LDS slots in wave order) and writes
// per-column-block partials, which delta_bwd_reduce_qk and
// delta_bwd_reduce_gb add over the column blocks and the value heads of a
// key head, again in a fixed order: results are bitwise reproducible.

#include <hip/hip_runtime.h>
#include <cmath>

#include "common.h"
#include "delta_rule.h"

namespace rglru {
namespace dbwd {

constexpr int kThreads = 512;  // 8 waves: one workgroup per CU, two waves per SIMD
constexpr int kTC = 16;  // tokens per chunk (the forward's checkpoint interval)

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  const float* ckpt;
  const void* d_o;
  const float* dh_last;
  void* dq;
  void* dk;
  void* dv;
  float* dg;
  float* dbeta;
  float* dh0;
  float* pdq;  // partials per column block: [NCB][tokens][Hv][Dk]
  float* pdk;
  float* pdg;  // [NCB][tokens][Hv] (GDN) or [NCB][tokens][Hv][Dk] (KDA)
  float* pdb;  // [NCB][tokens][Hv]
  const int32_t* cu;
  int64_t T, tokens, ck_slots;
  int Hk, Hv, Dk, Dv, grp;
  int n_cb;
  int n_blocks;
  int v_first;
  float scale;
};

__device__ __forceinline__ int xcd_remap(int id, int n) {
  const int q = n >> 3, r = n & 7, x = id & 7, pos = id >> 3;
  return x < r ? x * (q + 1) + pos : r * (q + 1) + (x - r) * q + pos;
}

template <int CTRL>
__device__ __forceinline__ float dpp_sum_step(float x) {
  // every control used here reads a valid lane, so no "old" value is needed (mov_dpp leaves it undefined)
  return x + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Lane layout of the backward: lane = rb * CPW + ciw, the CPW = 64 / LPC columns of a wave
// interleaved in the low lane bits, so that the sums over a wave's columns (18 per token) stay
// inside a quad or half-row (DPP), and only the sums over a column's rows (3 per token) cross
// DPP rows.

// sum over the columns of a wave (lanes with the same rb), every lane gets it; fixed order
template <int CPW>
__device__ __forceinline__ float column_sum(float x) {
  x = dpp_sum_step<0xB1>(x);                               // quad_perm [1,0,3,2]
  x = dpp_sum_step<0x4E>(x);                               // quad_perm [2,3,0,1]
  if constexpr (CPW == 8) x = dpp_sum_step<0x141>(x);      // row_half_mirror: the other quad of 8
  return x;
}

// x[lane] + x[lane ^ 16] (ROWS = 16) or x[lane] + x[lane ^ 32] (ROWS = 32) on every lane: the
// permlane swap of a register with a copy of itself leaves, in each lane, the pair of values the
// xor partner and the lane hold (a VALU exchange; a shuffle would go through LDS)
template <int ROWS>
__device__ __forceinline__ float swap_sum(float x) {
  const uint32_t u = __float_as_uint(x);
  if constexpr (ROWS == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
}

// sum over the rows of a column (lanes with the same ciw), every lane gets it; fixed order
template <int CPW>
__device__ __forceinline__ float row_sum(float x) {
  if constexpr (CPW == 4) x = dpp_sum_step<0x124>(x);      // row_ror 4
  x = dpp_sum_step<0x128>(x);                              // row_ror 8
  x = swap_sum<16>(x);
  x = swap_sum<32>(x);
  return x;
}

template <bool BF>
struct Io {
  static constexpr int VW = BF ? 8 : 4;
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
      return make_uint4(f32x2_to_bf16x2(f[0], f[1]), f32x2_to_bf16x2(f[2], f[3]), f32x2_to_bf16x2(f[4], f[5]),
                        f32x2_to_bf16x2(f[6], f[7]));
    } else {
      return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3]));
    }
  }
};

template <int LPC, int R, bool KDA, bool BF>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void delta_bwd_kernel(BwdArgs p) {
  using IO = Io<BF>;
  constexpr int VW = IO::VW;
  constexpr int DKP = LPC * R;
  constexpr int CW = kThreads / LPC;
  constexpr int KPT = DKP / VW;
  constexpr int VPT = CW / VW;
  constexpr int NW = kThreads / 64;
  static_assert(kTC * VPT <= kThreads && DKP % VW == 0 && CW % VW == 0 && R % 4 == 0, "tiling");

  __shared__ __align__(16) float sk[kTC][DKP];
  __shared__ __align__(16) float sq[kTC][DKP];
  __shared__ __align__(16) float sg[KDA ? kTC : 1][KDA ? DKP : 4];
  __shared__ float sgs[kTC], sb[kTC];
  __shared__ __align__(16) float sv[kTC][CW];
  __shared__ __align__(16) float sdo[kTC][CW];
  __shared__ __align__(16) float sdv[kTC][CW];
  // per-wave column sums of dq, dk (and dg, dbeta) for half a chunk, flushed every kTH tokens
  constexpr int kTH = kTC / 2;
  __shared__ float rq[NW][kTH][DKP];
  __shared__ float rk[NW][kTH][DKP];
  __shared__ float rg[NW][kTH][KDA ? DKP : 1];
  __shared__ float rb_[NW][kTH];

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
  const int wave = tid >> 6;
  constexpr int CPW = 64 / LPC;  // columns per wave
  const int rb = lane / CPW;      // row block of the column
  const int ciw = lane % CPW;     // column within the wave
  const int cl = wave * (64 / LPC) + ciw;
  const int col = cb * CW + cl;
  // lanes of columns past Dv start from a zero state and gradient and read v and do staged as
  // zero, so every term they add to the column sums is zero and needs no mask
  const bool col_ok = col < p.Dv;
  const int64_t st_base = ((int64_t)n * p.Hv + h) * p.Dk * p.Dv;
  auto st_index = [&](int row) -> int64_t {
    return st_base + (p.v_first ? (int64_t)col * p.Dk + row : (int64_t)row * p.Dv + col);
  };

  const char* qb = static_cast<const char*>(p.q);
  const char* kb = static_cast<const char*>(p.k);
  const char* vb = static_cast<const char*>(p.v);
  const char* dob = static_cast<const char*>(p.d_o);
  char* dvb = static_cast<char*>(p.dv);

  float G[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int row = rb * R + i;
    G[i] = (p.dh_last != nullptr && col_ok && row < p.Dk) ? p.dh_last[st_index(row)] : 0.0f;
  }

  const int64_t nch = (len + kTC - 1) / kTC;
  const int64_t ck0 = (int64_t)h * p.ck_slots + delta_ckpt_base(p.cu != nullptr, p.T, n, tok0);

  // A chunk's inputs are loaded into registers while the chunk after it is still being
  // processed (after its last reverse step), then converted into LDS: at most one piece of k and
  // q, one of v and do, NGK decays (KDA), beta and the decay (GDN) and the R checkpoint rows of
  // the lane's column per thread. Entries past the chunk's end or the head's size load as zero:
  // the staged k, q, v, do and beta are then zero and the decays exp(0) = 1.
  constexpr int NGK = (kTC * DKP + kThreads - 1) / kThreads;
  static_assert(kTC * KPT <= kThreads && kTC * VPT <= kThreads, "one staged piece per thread");
  uint4 rk4, rq4, rv4, ro4;
  float rgk[KDA ? NGK : 1], rbt, rgs, s0[R], s1[R];
  auto prefetch = [&](const int64_t c) {
    const int64_t t0 = tok0 + c * kTC;
    const int nt = (int)(len - c * kTC < kTC ? len - c * kTC : kTC);
    rk4 = rq4 = rv4 = ro4 = make_uint4(0u, 0u, 0u, 0u);
    {
      const int tt = tid / KPT, part = tid % KPT;
      if (tid < kTC * KPT && tt < nt && part * VW < p.Dk) {
        const int64_t e0 = ((t0 + tt) * p.Hk + kh) * p.Dk + part * VW;
        rk4 = *reinterpret_cast<const uint4*>(kb + e0 * IO::ES);
        rq4 = *reinterpret_cast<const uint4*>(qb + e0 * IO::ES);
      }
    }
    if constexpr (KDA) {
#pragma unroll
      for (int j = 0; j < NGK; ++j) {
        const int idx = tid + j * kThreads;
        const int tt = idx / DKP, d = idx % DKP;
        rgk[j] = (idx < kTC * DKP && tt < nt && d < p.Dk) ? p.g[((t0 + tt) * p.Hv + h) * p.Dk + d] : 0.f;
      }
    }
    {
      const int tt = tid / VPT, part = tid % VPT;
      const int c0 = cb * CW + part * VW;
      if (tid < kTC * VPT && tt < nt && c0 < p.Dv) {
        const int64_t e0 = ((t0 + tt) * p.Hv + h) * p.Dv + c0;
        rv4 = *reinterpret_cast<const uint4*>(vb + e0 * IO::ES);
        ro4 = *reinterpret_cast<const uint4*>(dob + e0 * IO::ES);
      }
    }
    {
      const bool ok = tid < nt;
      const int64_t e0 = (t0 + tid) * p.Hv + h;
      rbt = ok ? p.beta[e0] : 0.f;
      rgs = (!KDA && ok) ? p.g[e0] : 0.f;
    }
    // the states entering the chunk and its 9th token (checkpoint slots 2c and 2c + 1; the second
    // exists when the chunk has more than 8 tokens, else the second half is all padding and starts
    // from zero). Column-major slots: the lane's R rows of its column are contiguous (16-byte
    // loads; Dk is a multiple of 8, so a group of 4 rows is wholly inside it or wholly past it).
    static_assert(kTH == kDeltaCkpt, "one checkpoint per half chunk");
    const float* ck = p.ckpt + (ck0 + 2 * c) * p.Dk * p.Dv + (int64_t)col * p.Dk;
    const bool mid = nt > kTH;
#pragma unroll
    for (int i = 0; i < R; i += 4) {
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f), y = x;
      if (col_ok && rb * R + i < p.Dk) {
        x = *reinterpret_cast<const float4*>(ck + rb * R + i);
        if (mid) y = *reinterpret_cast<const float4*>(ck + (int64_t)p.Dk * p.Dv + rb * R + i);
      }
      s0[i] = x.x;
      s0[i + 1] = x.y;
      s0[i + 2] = x.z;
      s0[i + 3] = x.w;
      s1[i] = y.x;
      s1[i + 1] = y.y;
      s1[i + 2] = y.z;
      s1[i + 3] = y.w;
    }
  };
  auto stage = [&]() {
    if (tid < kTC * KPT) {
      const int tt = tid / KPT, part = tid % KPT;
      float fk[VW], fq[VW];
      IO::to_f32(rk4, fk);
      IO::to_f32(rq4, fq);
#pragma unroll
      for (int e = 0; e < VW; ++e) {
        sk[tt][part * VW + e] = fk[e];
        sq[tt][part * VW + e] = p.scale * fq[e];
      }
    }
    if constexpr (KDA) {
#pragma unroll
      for (int j = 0; j < NGK; ++j) {
        const int idx = tid + j * kThreads;
        if (idx < kTC * DKP) sg[idx / DKP][idx % DKP] = expf(rgk[j]);
      }
    }
    if (tid < kTC * VPT) {
      const int tt = tid / VPT, part = tid % VPT;
      float fv[VW], fo[VW];
      IO::to_f32(rv4, fv);
      IO::to_f32(ro4, fo);
#pragma unroll
      for (int e = 0; e < VW; ++e) {
        sv[tt][part * VW + e] = fv[e];
        sdo[tt][part * VW + e] = fo[e];
      }
    }
    if (tid < kTC) {
      sb[tid] = rbt;
      if constexpr (!KDA) sgs[tid] = expf(rgs);
    }
  };

  if (nch > 0) prefetch(nch - 1);
  for (int64_t c = nch - 1; c >= 0; --c) {
    const int64_t t0 = tok0 + c * kTC;
    const int nt = (int)(len - c * kTC < kTC ? len - c * kTC : kTC);
    stage();
    __syncthreads();

    // decayed states S~, errors e and writes u of one half chunk, recomputed forward from that
    // half's checkpoint: holding half a chunk is what lets two waves share a SIMD's registers
    constexpr int kHS = kTH;
    float hs[kHS][R], he[kHS], hu[kHS];
    auto recompute = [&](const int lo) {
      float s[R];
#pragma unroll
      for (int i = 0; i < R; ++i) s[i] = lo == 0 ? s0[i] : s1[i];
#pragma unroll
      for (int t = 0; t < kTC; ++t) {
        if (t >= lo && t < lo + kHS) {
          float kk[R];
#pragma unroll
          for (int i = 0; i < R; ++i) kk[i] = sk[t][rb * R + i];
#pragma unroll
          for (int i = 0; i < R; ++i) s[i] *= KDA ? sg[t][rb * R + i] : sgs[t];
          float a0 = 0.f, a1 = 0.f;
#pragma unroll
          for (int i = 0; i < R; i += 2) {
            a0 = fmaf(s[i], kk[i], a0);
            a1 = fmaf(s[i + 1], kk[i + 1], a1);
          }
          const float e = sv[t][cl] - row_sum<CPW>(a0 + a1);
          const float u = sb[t] * e;
#pragma unroll
          for (int i = 0; i < R; ++i) hs[t - lo][i] = s[i];
          he[t - lo] = e;
          hu[t - lo] = u;
#pragma unroll
          for (int i = 0; i < R; ++i) s[i] = fmaf(u, kk[i], s[i]);
        }
      }
    };

    // the reverse steps, the per-wave sums flushed to this column block's partials (waves
    // summed in order) after each half chunk
    auto rev = [&](const int t) {
        float kk[R], qq[R];
#pragma unroll
        for (int i = 0; i < R; ++i) {
          kk[i] = sk[t][rb * R + i];
          qq[i] = sq[t][rb * R + i];
        }
        const float dov = sdo[t][cl];
        const float dovs = p.scale * dov;
        const float bt = sb[t];
        float dqv[R], dkv[R], dgv[KDA ? R : 1];
#pragma unroll
        for (int i = 0; i < R; ++i) {
          G[i] = fmaf(qq[i], dov, G[i]);  // qq holds scale q
          dqv[i] = fmaf(kk[i], hu[t & (kHS - 1)], hs[t & (kHS - 1)][i]) * dovs;  // scale S do with S = S~ + k u
        }
        float d0 = 0.f, d1 = 0.f;
#pragma unroll
        for (int i = 0; i < R; i += 2) {
          d0 = fmaf(G[i], kk[i], d0);
          d1 = fmaf(G[i + 1], kk[i + 1], d1);
        }
        const float du = row_sum<CPW>(d0 + d1);
        const float da = -bt * du;
        float gs0 = 0.f;
#pragma unroll
        for (int i = 0; i < R; ++i) {
          dkv[i] = fmaf(G[i], hu[t & (kHS - 1)], hs[t & (kHS - 1)][i] * da);
          const float gt = fmaf(kk[i], da, G[i]);  // G~ = G - beta k du^T
          if constexpr (KDA) {
            dgv[i] = gt * hs[t & (kHS - 1)][i];
            G[i] = gt * sg[t][rb * R + i];
          } else {
            gs0 = fmaf(gt, hs[t & (kHS - 1)][i], gs0);
            G[i] = gt * sgs[t];
          }
        }
        if constexpr (!KDA) dgv[0] = row_sum<CPW>(gs0);
        float dbv = he[t & (kHS - 1)] * du;  // the same on every lane of the column
        if (rb == 0 && col_ok) sdv[t][cl] = bt * du;
        // sum over the wave's columns (fixed order), then one slot per wave
#pragma unroll
        for (int i = 0; i < R; ++i) {
          dqv[i] = column_sum<CPW>(dqv[i]);
          dkv[i] = column_sum<CPW>(dkv[i]);
        }
        if constexpr (KDA) {
#pragma unroll
          for (int i = 0; i < R; ++i) dgv[i] = column_sum<CPW>(dgv[i]);
        } else {
          dgv[0] = column_sum<CPW>(dgv[0]);
        }
        dbv = column_sum<CPW>(dbv);
        if (ciw == 0) {
#pragma unroll
          for (int i = 0; i < R; ++i) {
            rq[wave][t & (kTH - 1)][rb * R + i] = dqv[i];
            rk[wave][t & (kTH - 1)][rb * R + i] = dkv[i];
            if constexpr (KDA) rg[wave][t & (kTH - 1)][rb * R + i] = dgv[i];
          }
          if (rb == 0) {
            if constexpr (!KDA) rg[wave][t & (kTH - 1)][0] = dgv[0];
            rb_[wave][t & (kTH - 1)] = dbv;
          }
        }
    };
    auto flush = [&](const int lo) {
      __syncthreads();
      for (int idx = tid; idx < kTH * DKP; idx += kThreads) {
        const int tt = idx / DKP, d = idx % DKP;
        if (lo + tt < nt && d < p.Dk) {
          float aq = 0.f, ak = 0.f, ag = 0.f;
#pragma unroll
          for (int w = 0; w < NW; ++w) {
            aq += rq[w][tt][d];
            ak += rk[w][tt][d];
            if constexpr (KDA) ag += rg[w][tt][d];
          }
          const int64_t e0 = (((int64_t)cb * p.tokens + t0 + lo + tt) * p.Hv + h) * p.Dk + d;
          p.pdq[e0] = aq;
          p.pdk[e0] = ak;
          if constexpr (KDA) p.pdg[e0] = ag;
        }
      }
      if (tid < kTH && lo + tid < nt) {
        float ag = 0.f, ab = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          if constexpr (!KDA) ag += rg[w][tid][0];
          ab += rb_[w][tid];
        }
        const int64_t e0 = ((int64_t)cb * p.tokens + t0 + lo + tid) * p.Hv + h;
        if constexpr (!KDA) p.pdg[e0] = ag;
        p.pdb[e0] = ab;
      }
      __syncthreads();
    };
    // Every step runs, also over the tokens past nt in a sequence's last chunk: those are
    // staged with k = q = v = do = beta = 0 and decay 1, so their steps leave the state and the
    // gradient unchanged and their sums are never written; straight-line code keeps the
    // recomputed states in place (no merges of the register history at every token).
    recompute(kTC - kHS);
#pragma unroll
    for (int t = kTC - 1; t >= kTH; --t) rev(t);
    flush(kTH);
    recompute(0);
#pragma unroll
    for (int t = kTH - 1; t >= 0; --t) rev(t);
    if (c > 0) prefetch(c - 1);  // lands during the flush, the dv stores and the barrier
    flush(0);
    // dv
    {
      const int tt = tid / VPT, part = tid % VPT;
      const int c0 = cb * CW + part * VW;
      if (tid < kTC * VPT && tt < nt && c0 < p.Dv) {
        float f[VW];
#pragma unroll
        for (int e = 0; e < VW; ++e) f[e] = sdv[tt][part * VW + e];
        *reinterpret_cast<uint4*>(dvb + (((t0 + tt) * p.Hv + h) * p.Dv + c0) * IO::ES) = IO::from_f32(f);
      }
    }
    __syncthreads();
  }

  if (p.dh0 != nullptr && col_ok) {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int row = rb * R + i;
      if (row < p.Dk) p.dh0[st_index(row)] = G[i];
    }
  }
}

// dq, dk [tokens][Hk][Dk] (io dtype): the partials of every column block and every value head
// of the key head, in order. A thread takes 4 consecutive key channels (Dk is a multiple of 8,
// so they share a row and their partials are 16-byte aligned).
template <bool BF>
__global__ __launch_bounds__(256) void delta_bwd_reduce_qk(BwdArgs p) {
  const int64_t i4 = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int nd4 = p.Dk / 4;
  const int64_t total = p.tokens * p.Hk * nd4;
  if (i4 >= total) return;
  const int d = (int)(i4 % nd4) * 4;
  const int64_t r = i4 / nd4;
  const int kh = (int)(r % p.Hk);
  const int64_t tok = r / p.Hk;
  float4 aq = make_float4(0.f, 0.f, 0.f, 0.f), ak = aq;
  for (int hh = kh * p.grp; hh < (kh + 1) * p.grp; ++hh)
    for (int c = 0; c < p.n_cb; ++c) {
      const int64_t e0 = (((int64_t)c * p.tokens + tok) * p.Hv + hh) * p.Dk + d;
      const float4 x = *reinterpret_cast<const float4*>(p.pdq + e0);
      const float4 y = *reinterpret_cast<const float4*>(p.pdk + e0);
      aq.x += x.x; aq.y += x.y; aq.z += x.z; aq.w += x.w;
      ak.x += y.x; ak.y += y.y; ak.z += y.z; ak.w += y.w;
    }
  const int64_t o = r * p.Dk + d;
  if constexpr (BF) {
    // pairs of bf16 as 4-byte stores (dq and dk need only 4-byte alignment)
    uint32_t* dq = reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(p.dq) + o);
    uint32_t* dk = reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(p.dk) + o);
    dq[0] = f32x2_to_bf16x2(aq.x, aq.y);
    dq[1] = f32x2_to_bf16x2(aq.z, aq.w);
    dk[0] = f32x2_to_bf16x2(ak.x, ak.y);
    dk[1] = f32x2_to_bf16x2(ak.z, ak.w);
  } else {
    float* dq = static_cast<float*>(p.dq) + o;
    float* dk = static_cast<float*>(p.dk) + o;
    dq[0] = aq.x; dq[1] = aq.y; dq[2] = aq.z; dq[3] = aq.w;
    dk[0] = ak.x; dk[1] = ak.y; dk[2] = ak.z; dk[3] = ak.w;
  }
}

// dbeta [tokens][Hv] and dg [tokens][Hv] (GDN) or [tokens][Hv][Dk] (KDA), float32.
__global__ __launch_bounds__(256) void delta_bwd_reduce_gb(BwdArgs p, int kda) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t nb = p.tokens * p.Hv;
  const int64_t ng = kda ? nb * p.Dk : nb;
  if (i < ng) {
    float a = 0.f;
    for (int c = 0; c < p.n_cb; ++c) a += p.pdg[(int64_t)c * ng + i];
    p.dg[i] = a;
  }
  if (i < nb) {
    float a = 0.f;
    for (int c = 0; c < p.n_cb; ++c) a += p.pdb[(int64_t)c * nb + i];
    p.dbeta[i] = a;
  }
}

template <int LPC, int R, bool KDA, bool BF>
hipError_t launch(const BwdArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((delta_bwd_kernel<LPC, R, KDA, BF>), dim3(a.n_blocks), dim3(kThreads), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t nqk = a.tokens * a.Hk * (a.Dk / 4);
  if (nqk > 0) {
    hipLaunchKernelGGL((delta_bwd_reduce_qk<BF>), dim3((unsigned)((nqk + 255) / 256)), dim3(256), 0, st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t ng = a.tokens * a.Hv * (KDA ? a.Dk : 1);
    hipLaunchKernelGGL(delta_bwd_reduce_gb, dim3((unsigned)((ng + 255) / 256)), dim3(256), 0, st, a, KDA ? 1 : 0);
    e = hipGetLastError();
  }
  return e;
}

template <int LPC, int R>
hipError_t launch_dt(const BwdArgs& a, bool kda, bool bf, hipStream_t st) {
  if (kda) return bf ? launch<LPC, R, true, true>(a, st) : launch<LPC, R, true, false>(a, st);
  return bf ? launch<LPC, R, false, true>(a, st) : launch<LPC, R, false, false>(a, st);
}

struct Plan {
  int64_t N, n_cb, blocks, tokens, ck_slots;
  size_t pdq_off, pdk_off, pdg_off, pdb_off, bytes;
};

rglru_status_t plan(const rglru_delta_shape_t* sp, const int32_t* cu, int64_t n_seqs, Plan* pl) {
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
  if (cu != nullptr) {
    if (s.batch != 1 || n_seqs < 1 || n_seqs >= (int64_t(1) << 30)) return RGLRU_ERR_INVALID_ARGUMENT;
    N = n_seqs;
  }
  const int LPC = s.k_dim <= 64 ? 8 : 16;
  const int64_t n_cb = ceil_div(s.v_dim, kThreads / LPC);
  const int64_t blocks = N * s.v_heads * n_cb;
  if (blocks >= (int64_t(1) << 31)) return RGLRU_ERR_INVALID_ARGUMENT;
  // the backward's chunk registers hold R = 8 rows: Dk up to 128
  if (s.k_dim > 128 || s.k_dim % 8 != 0 || s.v_dim % 8 != 0) return RGLRU_ERR_UNSUPPORTED;
  const int64_t tokens = s.batch * s.length;
  if (tokens * s.k_heads * s.k_dim >= (int64_t(1) << 40)) return RGLRU_ERR_INVALID_ARGUMENT;
  const bool kda = s.decay == RGLRU_DELTA_KDA;
  const size_t nqk = (size_t)(n_cb * tokens * s.v_heads * s.k_dim);
  const size_t nb = (size_t)(n_cb * tokens * s.v_heads);
  pl->N = N;
  pl->n_cb = n_cb;
  pl->blocks = blocks;
  pl->tokens = tokens;
  pl->ck_slots = delta_ckpt_slots(cu != nullptr, s.length, s.batch, n_seqs);
  pl->pdq_off = 0;
  pl->pdk_off = round_up(nqk * 4, 256);
  pl->pdg_off = pl->pdk_off + round_up(nqk * 4, 256);
  pl->pdb_off = pl->pdg_off + round_up((kda ? nqk : nb) * 4, 256);
  pl->bytes = pl->pdb_off + round_up(nb * 4, 256);
  return RGLRU_OK;
}

}  // namespace dbwd
}  // namespace rglru

using namespace rglru;

extern "C" size_t rglru_delta_bwd_workspace_bytes(const rglru_delta_shape_t* shape, int64_t n_seqs) {
  dbwd::Plan pl;
  static const int32_t packed_marker = 0;
  if (dbwd::plan(shape, n_seqs > 0 ? &packed_marker : nullptr, n_seqs, &pl) != RGLRU_OK) return 0;
  return pl.bytes;
}

extern "C" rglru_status_t rglru_delta_rule_bwd(const rglru_delta_shape_t* shape, const int32_t* cu_seqlens,
                                               int64_t n_seqs, const void* q, const void* k, const void* v,
                                               const float* g, const float* beta, const float* ckpt,
                                               const void* d_o, const float* dh_last, void* dq, void* dk,
                                               void* dv, float* dg, float* dbeta, float* dh0, void* workspace,
                                               size_t workspace_bytes, void* stream) {
  dbwd::Plan pl;
  const rglru_status_t st = dbwd::plan(shape, cu_seqlens, n_seqs, &pl);
  if (st != RGLRU_OK) return st;
  const rglru_delta_shape_t& s = *shape;
  const bool kda = s.decay == RGLRU_DELTA_KDA;
  if (pl.tokens > 0 && (q == nullptr || k == nullptr || v == nullptr || g == nullptr || beta == nullptr ||
                        ckpt == nullptr || d_o == nullptr || dq == nullptr || dk == nullptr || dv == nullptr ||
                        dg == nullptr || dbeta == nullptr || workspace == nullptr))
    return RGLRU_ERR_INVALID_ARGUMENT;
  if (!aligned_to(q, 16) || !aligned_to(k, 16) || !aligned_to(v, 16) || !aligned_to(d_o, 16) ||
      !aligned_to(dv, 16) || !aligned_to(dq, 4) || !aligned_to(dk, 4) || !aligned_to(g, 4) ||
      !aligned_to(beta, 4) || !aligned_to(ckpt, 16) || !aligned_to(dh_last, 4) || !aligned_to(dg, 4) ||
      !aligned_to(dbeta, 4) || !aligned_to(dh0, 4) || !aligned_to(workspace, 256) || !aligned_to(cu_seqlens, 4))
    return RGLRU_ERR_MISALIGNED;
  if (pl.blocks == 0 || (pl.tokens == 0 && dh0 == nullptr)) return RGLRU_OK;
  if (pl.tokens > 0 && workspace_bytes < pl.bytes) return RGLRU_ERR_WORKSPACE_TOO_SMALL;
  char* ws = static_cast<char*>(workspace);
  dbwd::BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.beta = beta;
  a.ckpt = ckpt;
  a.d_o = d_o;
  a.dh_last = dh_last;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dg = dg;
  a.dbeta = dbeta;
  a.dh0 = dh0;
  a.pdq = reinterpret_cast<float*>(ws + pl.pdq_off);
  a.pdk = reinterpret_cast<float*>(ws + pl.pdk_off);
  a.pdg = reinterpret_cast<float*>(ws + pl.pdg_off);
  a.pdb = reinterpret_cast<float*>(ws + pl.pdb_off);
  a.cu = cu_seqlens;
  a.T = s.length;
  a.tokens = pl.tokens;
  a.ck_slots = pl.ck_slots;
  a.Hk = s.k_heads;
  a.Hv = s.v_heads;
  a.Dk = s.k_dim;
  a.Dv = s.v_dim;
  a.grp = s.v_heads / s.k_heads;
  a.n_cb = (int)pl.n_cb;
  a.n_blocks = (int)pl.blocks;
  a.v_first = s.state_v_first;
  a.scale = s.scale;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const bool bf = s.io_dtype == RGLRU_IO_BF16;
  const hipError_t e = s.k_dim <= 64 ? dbwd::launch_dt<8, 8>(a, kda, bf, hs) : dbwd::launch_dt<16, 8>(a, kda, bf, hs);
  return e == hipSuccess ? RGLRU_OK : RGLRU_ERR_HIP;
}
