// Gated delta rule forward, GDN chunk form, on bf16 MFMA (v_mfma_f32_32x32x16_bf16).
//
// The chunk algebra of the linear_attention reference page's
// chunk_gdn_reference (exact up to rounding, one unit-lower-triangular solve
// per chunk). Within a chunk of C = 64 tokens with in-chunk cumulative log
// decays Gc and the state S0 entering it:
//
//   A    = strictly lower part of diag(beta) (e^{Gc_i - Gc_j}) (K K^T)
//   T    = (I + A)^{-1}
//   W    = T diag(beta e^{Gc}) K,   Ut = T diag(beta) V           (the WY operands)
//   U    = Ut - W S0                                              (corrected writes)
//   P    = lower part (diagonal included) of (e^{Gc_i - Gc_j}) (Q K^T)
//   O    = scale (diag(e^{Gc}) Q S0 + P U)
//   S1   = e^{Gc_last} S0 + (diag(e^{Gc_last - Gc}) K)^T U
//
// Two launches. gdn_chunk_prep (one workgroup per chunk and value head, all
// in parallel) computes Gc, K K^T and Q K^T on MFMA, T by forward
// substitution in float32 on the vector ALUs, then W and Ut on MFMA, and
// writes -W, Ut, P, Gc and the decayed K^T to the workspace, each in the
// layout its consumer reads as MFMA fragments. gdn_chunk_state (one
// workgroup per value head and 32-column tile of the state, every column of
// S being independent) walks the chunks in order with its [Dk x 32] float32
// state tile held in MFMA accumulators: U = Ut + (-W) S0 and Q S0 on MFMA,
// then O and the state update. Its A operands come from global memory
// straight into registers, one chunk ahead; only the bf16 copies of the
// state tile and of U (the B operands) pass through LDS. MFMA operands are bf16 (q, k, v are bf16 already;
// T, W, Ut, P, U and the state's operand copy are rounded to bf16), every
// accumulation is float32, and the state itself stays float32.
//
// MFMA 32x32x16 lane layout used throughout (lane l, k-block kb = l / 32):
// A supplies row l % 32, elements k = 8 kb .. 8 kb + 7; B supplies column
// l % 32, the same k; accumulator register r holds row 8 (r / 4) + 4 kb +
// r % 4, column l % 32.

#include <hip/hip_runtime.h>
#include <cmath>

#include "common.h"
#include "delta_rule.h"

namespace rglru {
namespace dchunk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kC = 64;  // chunk length
constexpr int kThreads = 256;
constexpr int kTP = kC + 8;  // padded row (bf16 elements) of token-indexed LDS tiles
constexpr int kMaxDv = 256;
constexpr int kGS = 68;  // floats per chunk in gc_ws (16-byte multiple)

struct ChunkArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const float* g;
  const float* beta;
  const float* h0;
  uint16_t* o;
  float* h_last;
  // per (value head, chunk) = h * NCW + g, g counting the chunks of all sequences in order:
  uint16_t* w_ws;  // [64][Dk]                 bf16, -W
  uint16_t* u_ws;  // [Dv/32][2][64 lanes][16] bf16, Ut in accumulator order
  uint16_t* p_ws;  // [64][64]                 bf16, scale P
  float* gc_ws;    // [kGS]                    float32: scale e^{Gc_i} (i < 64), then e^{Gc_last} twice
  uint16_t* kt_ws; // [Dk][64]                 bf16, (diag(e^{Gc_last - Gc}) K)^T
  uint16_t* sink;  // 4 KiB that absorbs the output stores of rows past the end
  uint16_t* qs_ws; // [64][Dk]                 bf16, scale diag(e^Gc) Q
  const int32_t* cu;  // packed sequence offsets (n_seqs + 1), or NULL: B rows of T tokens
  int* cs;            // with cu: first chunk of each sequence (n_seqs + 1 entries), in the workspace
  int64_t T;
  int Hk, Hv, grp, Dv, NC, NV;
  int NCW;            // chunks per value head in the workspace: B * NC, or ceil(T / 64) + n_seqs
  int n_seqs;
  int n_blocks;
  int v_first;
  float scale;
};

__device__ __forceinline__ int xcd_remap(int id, int n) {
  const int q = n >> 3, r = n & 7, x = id & 7, pos = id >> 3;
  return x < r ? x * (q + 1) + pos : r * (q + 1) + (x - r) * q + pos;
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 ld8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ uint16_t h16(u32x4 v, int e) {
  return static_cast<uint16_t>(v[e >> 1] >> (16 * (e & 1)));
}

template <int CTRL>
__device__ __forceinline__ float dpp_sum_step(float x) {
  // every control used here reads a valid lane, so no "old" value is needed (mov_dpp leaves it undefined)
  return x + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

// A sequence's tokens [t0, t1) of the flattened [B * T] token axis and its chunks [c0, c1).
struct Seq {
  int64_t t0, t1;
  int c0, c1;
};

__device__ __forceinline__ Seq seq_info(const ChunkArgs& p, int n) {
  if (p.cu != nullptr) {
    int64_t a = p.cu[n], b = p.cu[n + 1];
    a = a < 0 ? 0 : (a > p.T ? p.T : a);
    b = b < a ? a : (b > p.T ? p.T : b);
    return {a, b, p.cs[n], p.cs[n + 1]};
  }
  return {(int64_t)n * p.T, (int64_t)(n + 1) * p.T, n * p.NC, (n + 1) * p.NC};
}

// The sequence holding chunk g (g below the total): the last n with cs[n] <= g.
__device__ __forceinline__ int seq_of_chunk(const ChunkArgs& p, int g) {
  if (p.cu == nullptr) return g / p.NC;
  int lo = 0, hi = p.n_seqs;  // cs[lo] <= g < cs[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (p.cs[mid] <= g) lo = mid; else hi = mid;
  }
  return lo;
}

// cs[n] = sum over m < n of ceil(len_m / 64) with the offsets clamped as in seq_info, cs[n_seqs]
// the total; each clamped to NCW (valid offsets never reach it; invalid ones, whose clamped
// sequences may overlap, then get unspecified but in-bounds results). One workgroup, the
// sequences in tiles of 1024 with a block-wide scan per tile, in 64-bit sums.
__global__ __launch_bounds__(1024) void gdn_chunk_map(ChunkArgs p) {
  __shared__ long long part[1024];
  __shared__ long long carry;
  const int tid = threadIdx.x;
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < p.n_seqs; base += 1024) {
    const int n = base + tid;
    long long v = 0;
    if (n < p.n_seqs) {
      int64_t a = p.cu[n], b = p.cu[n + 1];
      a = a < 0 ? 0 : (a > p.T ? p.T : a);
      b = b < a ? a : (b > p.T ? p.T : b);
      v = (b - a + kC - 1) / kC;
    }
    part[tid] = v;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {
      const long long add = tid >= d ? part[tid - d] : 0;
      __syncthreads();
      part[tid] += add;
      __syncthreads();
    }
    const long long c0 = carry;
    if (n < p.n_seqs) {
      const long long e = c0 + part[tid] - v;
      p.cs[n] = (int)(e < p.NCW ? e : p.NCW);
    }
    __syncthreads();
    if (tid == 1023) carry = c0 + part[1023];
    __syncthreads();
  }
  if (tid == 0) p.cs[p.n_seqs] = (int)(carry < p.NCW ? carry : p.NCW);
}

// ------------------------------------------------------------------ prep

// One workgroup per (chunk, value head). LDS region r1 holds K and Q (row-major) while K K^T
// and Q K^T run, then A (for the solve) and the two scaled copies of T.
template <int DK, int DVM>
__global__ __launch_bounds__(kThreads) void gdn_chunk_prep(ChunkArgs p) {
  constexpr int KP = DK + 8;
  constexpr int kKQ = 2 * kC * KP * 2;
  constexpr int kSTP = kC + 4;                    // padded row (floats) of the float32 T
  constexpr int kTB = 2 * kC * kTP * 2;           // Tw and Tu (bf16); the float32 T uses the same bytes
  static_assert(kC * kSTP * 4 <= kTB, "T in the Tw/Tu bytes");
  constexpr int kAT = kC * kC * 4 + kTB + 3 * 16 * 16 * 4;  // A, T (or Tw/Tu), three 16x16 temporaries
  constexpr int kR1 = kKQ > kAT ? kKQ : kAT;
  __shared__ __align__(16) unsigned char r1[kR1];
  __shared__ __align__(16) uint16_t sKt[DK][kTP];
  __shared__ __align__(16) uint16_t sVt[DVM][kTP];
  __shared__ float sG[kC], sGc[kC], sBeta[kC], sEg[kC], sEl[kC];
  uint16_t(*sK)[KP] = reinterpret_cast<uint16_t(*)[KP]>(r1);
  uint16_t(*sQ)[KP] = reinterpret_cast<uint16_t(*)[KP]>(r1 + kC * KP * 2);
  float(*sA)[kC] = reinterpret_cast<float(*)[kC]>(r1);  // row i: A[i][4 t + s] at [s * 16 + t]
  uint16_t(*sTw)[kTP] = reinterpret_cast<uint16_t(*)[kTP]>(r1 + kC * kC * 4);
  uint16_t(*sTu)[kTP] = reinterpret_cast<uint16_t(*)[kTP]>(r1 + kC * kC * 4 + kC * kTP * 2);
  float(*sT)[kSTP] = reinterpret_cast<float(*)[kSTP]>(r1 + kC * kC * 4);
  float(*sM)[16][16] = reinterpret_cast<float(*)[16][16]>(r1 + kC * kC * 4 + kTB);

  const int bid = xcd_remap(blockIdx.x, p.n_blocks);
  const int g = bid % p.NCW;
  const int h = bid / p.NCW, kh = h / p.grp;
  if (p.cu != nullptr && g >= p.cs[p.n_seqs]) return;  // the grid covers the most chunks any offsets give
  const Seq sq = seq_info(p, seq_of_chunk(p, g));
  const int64_t t0 = sq.t0 + (int64_t)(g - sq.c0) * kC;  // first token of the chunk (flattened)
  const int n = (int)(sq.t1 - t0 < kC ? sq.t1 - t0 : kC);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t chunk_id = (int64_t)h * p.NCW + g;

  // stage K and Q (row-major, K also transposed) and V (transposed), zero past the end; the
  // token index runs fastest across lanes so each transposed 2-byte write fills one row. Every
  // load is issued (at an in-bounds address) before the first LDS write.
  constexpr int NKG = kC * (DK / 8) / kThreads;
  constexpr int NVG = kC * (DVM / 8) / kThreads;
  const int r = tid & (kC - 1);
  const bool rok = r < n;
  const int64_t rowq = (t0 + (rok ? r : 0)) * p.Hk + kh;
  const int64_t rowv = (t0 + (rok ? r : 0)) * p.Hv + h;
  u32x4 kr[NKG], qr[NKG], vr[NVG];
#pragma unroll
  for (int j = 0; j < NKG; ++j) {
    const int part = (tid + kThreads * j) / kC;
    kr[j] = *reinterpret_cast<const u32x4*>(p.k + rowq * DK + part * 8);
    qr[j] = *reinterpret_cast<const u32x4*>(p.q + rowq * DK + part * 8);
  }
  const int vparts = p.Dv / 8;
#pragma unroll
  for (int j = 0; j < NVG; ++j) {
    const int part = (tid + kThreads * j) / kC;
    vr[j] = *reinterpret_cast<const u32x4*>(p.v + rowv * p.Dv + (part < vparts ? part : 0) * 8);
  }
  const int64_t eg = (t0 + (tid < n ? tid : 0)) * p.Hv + h;
  const float gv = p.g[eg], bv = p.beta[eg];
#pragma unroll
  for (int j = 0; j < NKG; ++j) {
    const int part = (tid + kThreads * j) / kC;
    const u32x4 z = {0u, 0u, 0u, 0u};
    const u32x4 kv = rok ? kr[j] : z, qv = rok ? qr[j] : z;
    *reinterpret_cast<u32x4*>(&sK[r][part * 8]) = kv;
    *reinterpret_cast<u32x4*>(&sQ[r][part * 8]) = qv;
#pragma unroll
    for (int e = 0; e < 8; ++e) sKt[part * 8 + e][r] = h16(kv, e);
  }
#pragma unroll
  for (int j = 0; j < NVG; ++j) {
    const int part = (tid + kThreads * j) / kC;
    const u32x4 z = {0u, 0u, 0u, 0u};
    const u32x4 vv = rok ? vr[j] : z;
    if (part < vparts) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sVt[part * 8 + e][r] = h16(vv, e);
    }
  }
  if (tid < kC) {
    sBeta[tid] = tid < n ? bv : 0.f;
    sG[tid] = tid < n ? gv : 0.f;
  }
  __syncthreads();
  if (tid < kC) {
    // inclusive prefix sum over the 64 lanes of wave 0 (log-step shuffles)
    float acc = sG[tid];
#pragma unroll
    for (int d = 1; d < kC; d <<= 1) {
      const float up = __shfl_up(acc, d, kC);
      if (tid >= d) acc += up;
    }
    sGc[tid] = acc;
  }
  __syncthreads();
  if (tid < kC) {
    const float eg = __expf(sGc[tid]);
    sEg[tid] = eg;
    sEl[tid] = __expf(sGc[kC - 1] - sGc[tid]);
    p.gc_ws[chunk_id * kGS + tid] = p.scale * eg;
  }
  if (tid == kC || tid == kC + 1) p.gc_ws[chunk_id * kGS + tid] = __expf(sGc[kC - 1]);  // two copies
  // scale diag(e^Gc) Q, from the staged registers, for the state pass's read-out
  {
    const float f = rok ? p.scale * __expf(sGc[r]) : 0.f;
    uint16_t* qw = p.qs_ws + (chunk_id * kC + r) * DK;
#pragma unroll
    for (int j = 0; j < NKG; ++j) {
      const int part = (tid + kThreads * j) / kC;
      u32x4 out;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        out[e] = f32x2_to_bf16x2(bf16_bits_to_f32(qr[j][e] & 0xFFFFu) * f, bf16_bits_to_f32(qr[j][e] >> 16) * f);
      *reinterpret_cast<u32x4*>(qw + part * 8) = out;
    }
  }
  __syncthreads();

  // K K^T and Q K^T, one 32x32 tile of each per wave
  const int ti = wave >> 1, tj = wave & 1;
  f32x16 akk = {}, aqk = {};
#pragma unroll
  for (int ks = 0; ks < DK / 16; ++ks) {
    const int kof = ks * 16 + (lane >> 5) * 8;
    const bf16x8 bk = ld8(&sK[tj * 32 + (lane & 31)][kof]);
    akk = mfma32(ld8(&sK[ti * 32 + (lane & 31)][kof]), bk, akk);
    aqk = mfma32(ld8(&sQ[ti * 32 + (lane & 31)][kof]), bk, aqk);
  }
  __syncthreads();  // K and Q are no longer read: A takes their place

  // A (strictly lower, scaled) to LDS; P (lower with diagonal, scaled) to the workspace
  {
    const int j = tj * 32 + (lane & 31);
    const float gj = sGc[j];
    uint16_t* pw = p.p_ws + chunk_id * kC * kC;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = ti * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
      const float dec = __expf(sGc[i] - gj);
      const float a = (j < i) ? sBeta[i] * dec * akk[r] : 0.f;
      sA[i][(j & 3) * 16 + (j >> 2)] = a;
      const float pv = (j <= i) ? p.scale * dec * aqk[r] : 0.f;
      pw[i * kC + j] = f32_to_bf16(pv);
    }
  }
  __syncthreads();

  // T = (I + A)^{-1} in 16 x 16 blocks. Diagonal blocks by forward substitution, one per wave:
  // T[i][j] = [i == j] - sum_{m < i} A[i][m] T[m][j] within the block; the 4 lanes of a quad
  // share column j, lane s holding rows 4 t + s of the block (t = 0 .. 3), a quad sum joining
  // their terms. Then the blocks below the diagonal by their distance d from it:
  // T[I][J] = -T[I][I] sum_{K = J}^{I - 1} A[I][K] T[K][J], with I = J + d.
  {
    const int w16 = wave * 16;
    const int j = w16 + (lane >> 2), s = lane & 3;
    float tr[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float4 a = *reinterpret_cast<const float4*>(&sA[w16 + i][s * 16 + 4 * wave]);
      float sum = fmaf(a.x, tr[0], a.y * tr[1]) + fmaf(a.z, tr[2], a.w * tr[3]);
      sum = dpp_sum_step<0xB1>(sum);
      sum = dpp_sum_step<0x4E>(sum);
      const float tij = (w16 + i == j ? 1.f : 0.f) - sum;
      if (s == (i & 3)) tr[i >> 2] = tij;
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) sT[w16 + 4 * t + s][j] = tr[t];
  }
  __syncthreads();
  {
    const int r = tid >> 4, cc = tid & 15;  // element (r, cc) of a 16 x 16 block
    // A[row][16 K + x] for x = 0 .. 15, from A's permuted rows
    auto arow = [&](int row, int K, float* x16) {
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const float4 v = *reinterpret_cast<const float4*>(&sA[row][s4 * 16 + 4 * K]);
        x16[s4] = v.x;
        x16[s4 + 4] = v.y;
        x16[s4 + 8] = v.z;
        x16[s4 + 12] = v.w;
      }
    };
#pragma unroll
    for (int d = 1; d < 4; ++d) {
      for (int J = 0; J + d < 4; ++J) {
        const int I = J + d;
        float m = 0.f;
        for (int K = J; K < I; ++K) {
          float x16[16];
          arow(16 * I + r, K, x16);
#pragma unroll
          for (int x = 0; x < 16; ++x) m = fmaf(x16[x], sT[16 * K + x][16 * J + cc], m);
        }
        sM[J][r][cc] = m;
      }
      __syncthreads();
      for (int J = 0; J + d < 4; ++J) {
        const int I = J + d;
        float t = 0.f;
#pragma unroll
        for (int x = 0; x < 16; ++x) t = fmaf(sT[16 * I + r][16 * I + x], sM[J][x][cc], t);
        sT[16 * I + r][16 * J + cc] = -t;
      }
      __syncthreads();
    }
  }
  // Tw = T diag(beta e^Gc), Tu = T diag(beta) in bf16, over the float32 T's bytes
  {
    const int m = tid >> 2, j0 = (tid & 3) * 16;
    float tv[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) tv[e] = (j0 + e <= m) ? sT[m][j0 + e] : 0.f;  // T is lower triangular
    __syncthreads();
    u32x4 w2[2], u2[2];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int ja = j0 + 2 * e, jb = ja + 1;
      const float ba = sBeta[ja], bb = sBeta[jb];
      w2[e >> 2][e & 3] = f32x2_to_bf16x2(tv[2 * e] * ba * sEg[ja], tv[2 * e + 1] * bb * sEg[jb]);
      u2[e >> 2][e & 3] = f32x2_to_bf16x2(tv[2 * e] * ba, tv[2 * e + 1] * bb);
    }
    *reinterpret_cast<u32x4*>(&sTw[m][j0]) = w2[0];
    *reinterpret_cast<u32x4*>(&sTw[m][j0 + 8]) = w2[1];
    *reinterpret_cast<u32x4*>(&sTu[m][j0]) = u2[0];
    *reinterpret_cast<u32x4*>(&sTu[m][j0 + 8]) = u2[1];
  }
  __syncthreads();

  // -W = -(T diag(beta e^Gc)) K  -> w_ws row-major [64][DK]
  {
    uint16_t* ww = p.w_ws + chunk_id * kC * DK;
    for (int tile = wave; tile < 2 * (DK / 32); tile += 4) {
      const int mi = tile & 1, td = tile >> 1;
      f32x16 acc = {};
#pragma unroll
      for (int ks = 0; ks < kC / 16; ++ks) {
        const int kof = ks * 16 + (lane >> 5) * 8;
        acc = mfma32(ld8(&sTw[mi * 32 + (lane & 31)][kof]), ld8(&sKt[td * 32 + (lane & 31)][kof]), acc);
      }
      const int d = td * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = mi * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        ww[i * DK + d] = f32_to_bf16(-acc[r]);
      }
    }
  }
  // Ut = (T diag(beta)) V -> u_ws in accumulator order
  for (int tile = wave; tile < 2 * p.NV; tile += 4) {
    const int mi = tile & 1, tv = tile >> 1;
    f32x16 acc = {};
#pragma unroll
    for (int ks = 0; ks < kC / 16; ++ks) {
      const int kof = ks * 16 + (lane >> 5) * 8;
      acc = mfma32(ld8(&sTu[mi * 32 + (lane & 31)][kof]), ld8(&sVt[tv * 32 + (lane & 31)][kof]), acc);
    }
    uint16_t* uw = p.u_ws + (((chunk_id * p.NV + tv) * 2 + mi) * 64 + lane) * 16;
    u32x4 lo, hi;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      lo[e] = f32x2_to_bf16x2(acc[2 * e], acc[2 * e + 1]);
      hi[e] = f32x2_to_bf16x2(acc[8 + 2 * e], acc[8 + 2 * e + 1]);
    }
    *reinterpret_cast<u32x4*>(uw) = lo;
    *reinterpret_cast<u32x4*>(uw + 8) = hi;
  }
  // (e^{Gc_last - Gc} K)^T -> kt_ws row-major [DK][64]
  {
    uint16_t* kw = p.kt_ws + chunk_id * DK * kC;
    for (int idx = tid; idx < DK * 8; idx += kThreads) {
      const int d = idx >> 3, part = idx & 7;
      const u32x4 kv = *reinterpret_cast<const u32x4*>(&sKt[d][part * 8]);
      u32x4 out;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = part * 8 + 2 * e;
        out[e] = f32x2_to_bf16x2(bf16_bits_to_f32(kv[e] & 0xFFFFu) * sEl[m], bf16_bits_to_f32(kv[e] >> 16) * sEl[m + 1]);
      }
      *reinterpret_cast<u32x4*>(kw + d * kC + part * 8) = out;
    }
  }
}

// ------------------------------------------------------------------ state pass

// The state pass: one workgroup of 8 waves per (value head, 32-column tile of the state),
// walking the chunks in order. Roles, each in a loop of its own with the same two barriers
// per chunk:
//   waves 0, 1 (U): U = U~ + (-W) S for token rows 32 w .. 32 w + 31, to LDS as bf16;
//   waves 2, 3 (O): scale e^Gc Q S, then + scale P U, for those rows, to LDS, then out;
//   waves 4 .. 4 + Dk/32 - 1 (S): state rows 32 (w - 4) .. + 31 in MFMA accumulators,
//     S = e^{Gc_last} S + (e^{Gc_last - Gc} K)^T U, and their bf16 copy in LDS.
// A operands come from global memory straight into registers one chunk ahead; each role's
// loop issues the same loads every chunk, so the compiler's count of outstanding loads is
// exact and the prefetch is not waited for early. B operands (the state's and U's bf16
// copies) pass through LDS.
constexpr int kStateThreads = 512;

template <int DK>
__global__ __launch_bounds__(kStateThreads) void gdn_chunk_state(ChunkArgs p) {
  constexpr int KP = DK + 8;
  constexpr int ST = DK / 32;
  constexpr int KS = DK / 16;
  __shared__ __align__(16) uint16_t sS[32][KP];   // bf16 state tile, [column][key]
  __shared__ __align__(16) uint16_t sU[32][kTP];  // bf16 U, [column][token]
  __shared__ __align__(16) uint16_t sO[kC][40];   // bf16 outputs, [token][column]

  const int bid = xcd_remap(blockIdx.x, p.n_blocks);
  const int tv = bid % p.NV;
  const int bh = bid / p.NV;  // sequence * Hv + value head
  const int h = bh % p.Hv, seq = bh / p.Hv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = tv * 32 + (lane & 31);
  const int kb8 = (lane >> 5) * 8;
  const int64_t st_base = (int64_t)bh * DK * p.Dv;
  const Seq sq = seq_info(p, seq);
  const int NC = sq.c1 - sq.c0;                      // this sequence's chunks
  const int64_t cid0 = (int64_t)h * p.NCW + sq.c0;   // workspace index of its first chunk

  // the output rows of one chunk, from LDS, by the S waves (idle until U is complete):
  // thread -> token row / 4, 8 columns at 8 (thread % 4); rows past the end go to the sink
  auto store_out = [&](int c) {
    const int st = tid - 256;
    const int orow = st >> 2, ocol = (st & 3) * 8;
    const int64_t t0 = sq.t0 + (int64_t)c * kC;
    const u32x4 val = *reinterpret_cast<const u32x4*>(&sO[orow][ocol]);
    uint16_t* dst = t0 + orow < sq.t1 ? p.o + ((t0 + orow) * p.Hv + h) * p.Dv + tv * 32 + ocol : p.sink + st * 8;
    *reinterpret_cast<u32x4*>(dst) = val;
  };
  auto bsS = [&](int ks) { return ld8(&sS[lane & 31][ks * 16 + kb8]); };
  auto bsU = [&](int ks) { return ld8(&sU[lane & 31][ks * 16 + kb8]); };

  if (wave < 4) {
    const bool is_u = wave < 2;
    const int ti = wave & 1;
    const int arow = ti * 32 + (lane & 31);
    struct Ops {
      u32x4 a[KS];
      u32x4 x[4];  // U waves: U~ (two registers used); O waves: rows of P
    };
    auto load = [&](int c, Ops& o) {
      const int64_t cid = cid0 + c;
      const uint16_t* ab = (is_u ? p.w_ws : p.qs_ws) + (cid * kC + arow) * DK + kb8;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) o.a[ks] = *reinterpret_cast<const u32x4*>(ab + ks * 16);
      const uint16_t* xb = is_u ? p.u_ws + (((cid * p.NV + tv) * 2 + ti) * 64 + lane) * 16
                                : p.p_ws + (cid * kC + arow) * kC + kb8;
      const int xs = is_u ? 8 : 16;
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4) o.x[k4] = *reinterpret_cast<const u32x4*>(xb + (k4 & (is_u ? 1 : 3)) * xs);
    };
    // pf: the chunk whose operands are loaded into nx once this wave's part before barrier (1) is
    // done (off the corrected writes' critical path)
    auto step = [&](int c, const Ops& o, int pf, Ops& nx) {
      f32x16 acc = {};
      if (is_u) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] = bf16_bits_to_f32(o.x[0][e] & 0xFFFFu);
          acc[2 * e + 1] = bf16_bits_to_f32(o.x[0][e] >> 16);
          acc[8 + 2 * e] = bf16_bits_to_f32(o.x[1][e] & 0xFFFFu);
          acc[8 + 2 * e + 1] = bf16_bits_to_f32(o.x[1][e] >> 16);
        }
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) acc = mfma32(__builtin_bit_cast(bf16x8, o.a[ks]), bsS(ks), acc);
      if (is_u) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int i = ti * 32 + g4 * 8 + (lane >> 5) * 4;
          *reinterpret_cast<u32x2*>(&sU[lane & 31][i]) =
              u32x2{f32x2_to_bf16x2(acc[4 * g4], acc[4 * g4 + 1]), f32x2_to_bf16x2(acc[4 * g4 + 2], acc[4 * g4 + 3])};
        }
      }
      load(pf, nx);
      __syncthreads();  // (1) U complete; the state tile is no longer read
      if (!is_u) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) acc = mfma32(__builtin_bit_cast(bf16x8, o.x[ks]), bsU(ks), acc);
#pragma unroll
        for (int r = 0; r < 16; ++r)
          sO[ti * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3)][lane & 31] = f32_to_bf16(acc[r]);
      }
      __syncthreads();  // (2) outputs and the new state tile written; U no longer read
    };
    Ops o0, o1;
    if (NC > 0) load(0, o0);
    __syncthreads();  // (0) initial state tile written
    for (int c = 0; c < NC; c += 2) {
      step(c, o0, c + 1 < NC ? c + 1 : c, o1);
      if (c + 1 >= NC) break;
      step(c + 1, o1, c + 2 < NC ? c + 2 : c + 1, o0);
    }
  } else {
    const int sw = wave - 4;
    const bool owns = sw < ST;
    const int kw = owns ? sw : 0;
    f32x16 s_acc = {};
    auto srow = [&](int r) { return kw * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3); };
    auto sidx = [&](int d) -> int64_t {
      return st_base + (p.v_first ? (int64_t)col * DK + d : (int64_t)d * p.Dv + col);
    };
    if (p.h0 != nullptr) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s_acc[r] = p.h0[sidx(srow(r))];
    }
    __builtin_amdgcn_s_waitcnt(0);  // the initial state is in registers before the loop
    auto write_sS = [&]() {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = kw * 32 + g4 * 8 + (lane >> 5) * 4;
        *reinterpret_cast<u32x2*>(&sS[lane & 31][d]) = u32x2{f32x2_to_bf16x2(s_acc[4 * g4], s_acc[4 * g4 + 1]),
                                                             f32x2_to_bf16x2(s_acc[4 * g4 + 2], s_acc[4 * g4 + 3])};
      }
    };
    if (owns) write_sS();
    struct Ops {
      u32x4 kt[4];
      float el;  // e^{Gc_last}
    };
    auto load = [&](int c, Ops& o) {
      const int64_t cid = cid0 + c;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        o.kt[ks] = *reinterpret_cast<const u32x4*>(p.kt_ws + (cid * DK + kw * 32 + (lane & 31)) * kC + ks * 16 + kb8);
      // a vector load (its address depends on the lane: either of the two copies), issued here with
      // the other prefetches rather than reloaded at its use
      o.el = p.gc_ws[cid * kGS + kC + (lane & 1)];
    };
    auto step = [&](int c, const Ops& o) {
      if (c > 0) store_out(c - 1);
      __syncthreads();  // (1) U complete
      if (owns) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s_acc[r] *= o.el;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) s_acc = mfma32(__builtin_bit_cast(bf16x8, o.kt[ks]), bsU(ks), s_acc);
        write_sS();
      }
      __syncthreads();  // (2)
    };
    Ops o0, o1;
    if (NC > 0) load(0, o0);
    __syncthreads();  // (0)
    for (int c = 0; c < NC; c += 2) {
      load(c + 1 < NC ? c + 1 : c, o1);
      step(c, o0);
      if (c + 1 >= NC) break;
      load(c + 2 < NC ? c + 2 : c + 1, o0);
      step(c + 1, o1);
    }
    if (NC > 0) store_out(NC - 1);
    if (owns && p.h_last != nullptr) {
#pragma unroll
      for (int r = 0; r < 16; ++r) p.h_last[sidx(srow(r))] = s_acc[r];
    }
  }
}

template <int DK>
hipError_t launch(ChunkArgs a, int64_t prep_blocks, int64_t state_blocks, hipStream_t st) {
  if (a.cu != nullptr) {
    hipLaunchKernelGGL(gdn_chunk_map, dim3(1), dim3(1024), 0, st, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (prep_blocks > 0) {
    a.n_blocks = (int)prep_blocks;
    if (a.Dv <= 128)
      hipLaunchKernelGGL((gdn_chunk_prep<DK, 128>), dim3((unsigned)prep_blocks), dim3(kThreads), 0, st, a);
    else
      hipLaunchKernelGGL((gdn_chunk_prep<DK, kMaxDv>), dim3((unsigned)prep_blocks), dim3(kThreads), 0, st, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  a.n_blocks = (int)state_blocks;
  hipLaunchKernelGGL(gdn_chunk_state<DK>, dim3((unsigned)state_blocks), dim3(kStateThreads), 0, st, a);
  return hipGetLastError();
}

struct Plan {
  int64_t NC, NV, NCW, N, prep_blocks, state_blocks;
  size_t w_off, u_off, p_off, g_off, kt_off, qs_off, cs_off, sink_off, bytes;
};

// Validates the shape for the chunk form; fills the workspace plan. n_seqs = 0: B rows of T
// tokens; n_seqs >= 1: that many packed sequences (B = 1).
rglru_status_t plan(const rglru_delta_shape_t* sp, int64_t n_seqs, Plan* pl) {
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
  if (n_seqs < 0 || (n_seqs > 0 && (s.batch != 1 || n_seqs >= (int64_t(1) << 30)))) return RGLRU_ERR_INVALID_ARGUMENT;
  if (s.decay != RGLRU_DELTA_GDN || s.io_dtype != RGLRU_IO_BF16 || (s.k_dim != 64 && s.k_dim != 128) ||
      s.v_dim % 32 != 0 || s.v_dim > kMaxDv)
    return RGLRU_ERR_UNSUPPORTED;
  const int64_t NC = ceil_div(s.length, kC), NV = s.v_dim / 32;
  const int64_t N = n_seqs > 0 ? n_seqs : s.batch;
  const int64_t NCW = n_seqs > 0 ? NC + n_seqs : s.batch * NC;  // each sequence adds at most one partial chunk
  if (NCW * s.v_heads >= (int64_t(1) << 31) || N * s.v_heads * NV >= (int64_t(1) << 31))
    return RGLRU_ERR_INVALID_ARGUMENT;
  const size_t chunks = (size_t)(NCW * s.v_heads);
  pl->NC = NC;
  pl->NV = NV;
  pl->NCW = NCW;
  pl->N = N;
  pl->prep_blocks = NCW * s.v_heads;
  pl->state_blocks = N * s.v_heads * NV;
  pl->w_off = 0;
  pl->u_off = round_up(pl->w_off + chunks * kC * s.k_dim * 2, 256);
  pl->p_off = round_up(pl->u_off + chunks * kC * s.v_dim * 2, 256);
  pl->g_off = round_up(pl->p_off + chunks * kC * kC * 2, 256);
  pl->kt_off = round_up(pl->g_off + chunks * kGS * 4, 256);
  pl->qs_off = round_up(pl->kt_off + chunks * kC * s.k_dim * 2, 256);
  pl->cs_off = round_up(pl->qs_off + chunks * kC * s.k_dim * 2, 256);
  pl->sink_off = round_up(pl->cs_off + (size_t)(n_seqs + 1) * 4, 256);
  pl->bytes = pl->sink_off + 4096;
  return RGLRU_OK;
}

}  // namespace dchunk
}  // namespace rglru

using namespace rglru;

extern "C" size_t rglru_delta_chunk_workspace_bytes(const rglru_delta_shape_t* shape, int64_t n_seqs) {
  dchunk::Plan pl;
  if (dchunk::plan(shape, n_seqs, &pl) != RGLRU_OK) return 0;
  return pl.bytes;
}

extern "C" rglru_status_t rglru_delta_chunk_fwd(const rglru_delta_shape_t* shape, const int32_t* cu_seqlens,
                                                int64_t n_seqs, const void* q, const void* k, const void* v,
                                                const float* g, const float* beta, const float* h0, void* o,
                                                float* h_last, void* workspace, size_t workspace_bytes,
                                                void* stream) {
  if (cu_seqlens == nullptr) n_seqs = 0;
  else if (n_seqs < 1) return RGLRU_ERR_INVALID_ARGUMENT;
  dchunk::Plan pl;
  const rglru_status_t st = dchunk::plan(shape, n_seqs, &pl);
  if (st != RGLRU_OK) return st;
  const rglru_delta_shape_t& s = *shape;
  const int64_t tokens = s.batch * s.length;
  if (tokens > 0 && (q == nullptr || k == nullptr || v == nullptr || g == nullptr || beta == nullptr ||
                     o == nullptr))
    return RGLRU_ERR_INVALID_ARGUMENT;
  // the workspace holds the chunks' operands and, for packed sequences, the chunk map; with no
  // tokens and no packed sequences there are no chunks and it is not touched
  const bool needs_ws = tokens > 0 || cu_seqlens != nullptr;
  if (needs_ws && workspace == nullptr) return RGLRU_ERR_INVALID_ARGUMENT;
  if (!aligned_to(q, 16) || !aligned_to(k, 16) || !aligned_to(v, 16) || !aligned_to(o, 2) ||
      !aligned_to(g, 4) || !aligned_to(beta, 4) || !aligned_to(h0, 4) || !aligned_to(h_last, 4) ||
      !aligned_to(workspace, 256) || !aligned_to(cu_seqlens, 4))
    return RGLRU_ERR_MISALIGNED;
  if (pl.N * s.v_heads == 0 || (tokens == 0 && h_last == nullptr)) return RGLRU_OK;
  if (needs_ws && workspace_bytes < pl.bytes) return RGLRU_ERR_WORKSPACE_TOO_SMALL;
  if (tokens == 0) pl.prep_blocks = 0;
  char* ws = static_cast<char*>(workspace);
  dchunk::ChunkArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.g = g;
  a.beta = beta;
  a.h0 = h0;
  a.o = static_cast<uint16_t*>(o);
  a.h_last = h_last;
  a.w_ws = reinterpret_cast<uint16_t*>(ws + pl.w_off);
  a.u_ws = reinterpret_cast<uint16_t*>(ws + pl.u_off);
  a.p_ws = reinterpret_cast<uint16_t*>(ws + pl.p_off);
  a.gc_ws = reinterpret_cast<float*>(ws + pl.g_off);
  a.kt_ws = reinterpret_cast<uint16_t*>(ws + pl.kt_off);
  a.qs_ws = reinterpret_cast<uint16_t*>(ws + pl.qs_off);
  a.cs = reinterpret_cast<int*>(ws + pl.cs_off);
  a.sink = reinterpret_cast<uint16_t*>(ws + pl.sink_off);
  a.cu = cu_seqlens;
  a.T = s.length;
  a.Hk = s.k_heads;
  a.Hv = s.v_heads;
  a.grp = s.v_heads / s.k_heads;
  a.Dv = s.v_dim;
  a.NC = (int)pl.NC;
  a.NV = (int)pl.NV;
  a.NCW = (int)pl.NCW;
  a.n_seqs = (int)n_seqs;
  a.n_blocks = 0;
  a.v_first = s.state_v_first;
  a.scale = s.scale;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const hipError_t e = s.k_dim == 64 ? dchunk::launch<64>(a, pl.prep_blocks, pl.state_blocks, hs)
                                     : dchunk::launch<128>(a, pl.prep_blocks, pl.state_blocks, hs);
  return e == hipSuccess ? RGLRU_OK : RGLRU_ERR_HIP;
}
