// Block-diagonal gate projections on MFMA (gfx950), forward and backward.
//
// The Fattori comparison page has the caller compute two BlockDiagonalLinear
// gate projections of the recurrent input before the fused operator; here
// both gates of one 256-wide block are produced from a single read of x:
//   gate_g[:, blk] = x[:, blk] @ w_g[blk] + b_g[blk]      (w_g[blk] read as [in, out])
// Backward:
//   dx[:, blk]     = dx_in[:, blk] + sum_g dgate_g[:, blk] @ w_g[blk]^T
//   dw_g[blk]      = x[:, blk]^T @ dgate_g[:, blk]
//   db_g[blk]      = column sums of dgate_g[:, blk]
// bf16 operands, float32 accumulation (v_mfma_f32_16x16x32_bf16: A 16x32,
// B 32x16; lane l holds row/column l%16 and k = (l/16)*8 .. +7; D lane l holds
// column l%16, rows (l/16)*4 .. +3).
//
// Forward and dx kernels: a workgroup (4 waves) owns one half (128 rows of
// the MFMA M dimension) of one block for both gates, stages those weights in
// LDS once (the forward stores them transposed so that every fragment is 16
// contiguous bytes), and then walks token tiles of 128 (32 per wave),
// prefetching the next tile's token fragments from HBM while it multiplies.
// dW kernel: K runs over tokens, so 32-token slabs of x and of the gate
// gradient are staged transposed in LDS (double-buffered); each workgroup owns
// one (block, gate) and a contiguous token range, keeps the whole 256x256
// float32 block in accumulators, and writes a partial that a second kernel
// sums over token ranges in a fixed order (deterministic).
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.h"

namespace rglru {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBS = 256;          // block size (in = out = 256)
constexpr int kHalf = 128;        // staged rows per workgroup
constexpr int kPad = 264;         // LDS row stride in elements (528 B: conflict-free 16 B reads)
constexpr int kWaves = 4;
constexpr int kNT = 32;           // tokens per wave per tile
constexpr int kTileT = kWaves * kNT;
constexpr int kKSteps = kBS / 32;
constexpr int kSlab = 32;         // tokens per dW k-step
constexpr int kSlabPad = 40;      // LDS row stride of a transposed slab (80 B: conflict-free)

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ u32x4 load16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }

__device__ __forceinline__ uint32_t pack2(float lo, float hi) { return f32x2_to_bf16x2(lo, hi); }

__device__ __forceinline__ float bf(uint16_t v) { return bf16_bits_to_f32(v); }

// token fragments of one tile: [n-tile 0..1][k-step 0..7]
struct TokFrags {
  u32x4 f[2][kKSteps];
};

// Loads the B fragments of 32 tokens: row (token) t0 + nt*16 + l%16, columns
// col0 + ks*32 + (l/16)*8 .. +7 of a [T, ld] bf16 matrix (zeros past T).
__device__ __forceinline__ void load_tok_frags(TokFrags& fr, const uint16_t* m, long long ld, long long T,
                                               long long t0, int col0, int lane) {
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const long long t = t0 + nt * 16 + (lane & 15);
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
      if (t < T) {
        fr.f[nt][ks] = load16(m + t * ld + col0 + ks * 32 + (lane >> 4) * 8);
      } else {
        fr.f[nt][ks] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
}

// acc[mt][nt] += Wst[mt-tile rows][k] * frags over the 8 k-steps. The A
// fragments of the next k-step are read from LDS while the current one
// multiplies; the scheduling barrier keeps the compiler from hoisting every
// LDS read of the tile at once (which would exhaust the register file).
__device__ __forceinline__ void mma_tile(f32x4 (&acc)[8][2], const uint16_t (*w)[kPad], const TokFrags& fr,
                                         int lane) {
  bf16x8 a[2][8];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
    a[0][mt] = as_bf16x8(*reinterpret_cast<const u32x4*>(&w[mt * 16 + (lane & 15)][(lane >> 4) * 8]));
  }
#pragma unroll
  for (int ks = 0; ks < kKSteps; ++ks) {
    const int c = ks & 1;
    if (ks + 1 < kKSteps) {
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        a[c ^ 1][mt] = as_bf16x8(
            *reinterpret_cast<const u32x4*>(&w[mt * 16 + (lane & 15)][(ks + 1) * 32 + (lane >> 4) * 8]));
      }
    }
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      acc[mt][0] = mfma(a[c][mt], as_bf16x8(fr.f[0][ks]), acc[mt][0]);
      acc[mt][1] = mfma(a[c][mt], as_bf16x8(fr.f[1][ks]), acc[mt][1]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

struct ProjFwdArgs {
  const uint16_t* x;
  const uint16_t* w[2];
  const uint16_t* bias[2];
  uint16_t* out[2];
  long long T;
  int Wd;
  int splits;
};

__global__ __launch_bounds__(256) void proj_fwd_kernel(ProjFwdArgs p) {
  __shared__ __attribute__((aligned(16))) uint16_t s_w[2][kHalf][kPad];   // [gate][out][in]
  __shared__ float s_bias[2][kHalf];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kb = blockIdx.y >> 1;
  const int half = blockIdx.y & 1;
  const int col0 = kb * kBS;                 // first column of this block in x and the outputs
  const int out0 = half * kHalf;             // first output column (within the block) owned here

  // stage w_g[kb][in][out0 .. out0+127] transposed: s_w[g][out][in]
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const uint16_t* wb = p.w[g] + static_cast<long long>(kb) * kBS * kBS;
    for (int it = tid; it < (kBS / 2) * (kHalf / 8); it += 256) {
      const int in = (it / (kHalf / 8)) * 2;
      const int o = (it % (kHalf / 8)) * 8;
      const u32x4 r0 = load16(wb + in * kBS + out0 + o);
      const u32x4 r1 = load16(wb + (in + 1) * kBS + out0 + o);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t lo = (r0[j >> 1] >> ((j & 1) * 16)) & 0xFFFFu;
        const uint32_t hi = (r1[j >> 1] >> ((j & 1) * 16)) & 0xFFFFu;
        *reinterpret_cast<uint32_t*>(&s_w[g][o + j][in]) = lo | (hi << 16);
      }
    }
  }
  // bias of the 128 output columns owned here
  for (int it = tid; it < 2 * kHalf; it += 256) {
    const int g = it / kHalf;
    const int o = it % kHalf;
    s_bias[g][o] = p.bias[g] != nullptr ? bf(p.bias[g][col0 + out0 + o]) : 0.0f;
  }
  __syncthreads();

  const long long n_tiles = (p.T + kTileT - 1) / kTileT;
  long long tile = blockIdx.x;
  if (tile >= n_tiles) return;
  TokFrags cur;
  load_tok_frags(cur, p.x, p.Wd, p.T, tile * kTileT + wave * kNT, col0, lane);
  for (; tile < n_tiles; tile += p.splits) {
    const long long t0 = tile * kTileT + wave * kNT;
    TokFrags nxt;
    const long long ntile = tile + p.splits;
    if (ntile < n_tiles) load_tok_frags(nxt, p.x, p.Wd, p.T, ntile * kTileT + wave * kNT, col0, lane);
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      f32x4 acc[8][2];
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        acc[mt][0] = f32x4{0.f, 0.f, 0.f, 0.f};
        acc[mt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      mma_tile(acc, s_w[g], cur, lane);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const long long t = t0 + nt * 16 + (lane & 15);
        if (t < p.T) {
          uint16_t* orow = p.out[g] + t * p.Wd + col0 + out0 + (lane >> 4) * 4;
#pragma unroll
          for (int mt = 0; mt < 8; ++mt) {
            const float* bb = &s_bias[g][mt * 16 + (lane >> 4) * 4];
            u32x2 v;
            v[0] = pack2(acc[mt][nt][0] + bb[0], acc[mt][nt][1] + bb[1]);
            v[1] = pack2(acc[mt][nt][2] + bb[2], acc[mt][nt][3] + bb[3]);
            *reinterpret_cast<u32x2*>(orow + mt * 16) = v;
          }
        }
      }
    }
    if (ntile < n_tiles) cur = nxt;
  }
}

struct ProjDxArgs {
  const uint16_t* w[2];
  const uint16_t* dg[2];
  const uint16_t* dx_in;
  uint16_t* dx_out;
  long long T;
  int Wd;
  int splits;
};

// dx rows in0 .. in0+127 of block kb: A = w_g[kb][in][out] (natural layout), B = dgate_g tokens.
__global__ __launch_bounds__(256) void proj_dx_kernel(ProjDxArgs p) {
  __shared__ __attribute__((aligned(16))) uint16_t s_w[2][kHalf][kPad];   // [gate][in][out]
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kb = blockIdx.y >> 1;
  const int half = blockIdx.y & 1;
  const int col0 = kb * kBS;
  const int in0 = half * kHalf;

#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const uint16_t* wb = p.w[g] + static_cast<long long>(kb) * kBS * kBS;
    for (int it = tid; it < kHalf * (kBS / 8); it += 256) {
      const int r = it / (kBS / 8);
      const int o = (it % (kBS / 8)) * 8;
      *reinterpret_cast<u32x4*>(&s_w[g][r][o]) = load16(wb + (in0 + r) * kBS + o);
    }
  }
  __syncthreads();

  const long long n_tiles = (p.T + kTileT - 1) / kTileT;
  for (long long tile = blockIdx.x; tile < n_tiles; tile += p.splits) {
    const long long t0 = tile * kTileT + wave * kNT;
    f32x4 acc[8][2];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      acc[mt][0] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc[mt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    TokFrags fr[2];
    load_tok_frags(fr[0], p.dg[0], p.Wd, p.T, t0, col0, lane);
    load_tok_frags(fr[1], p.dg[1], p.Wd, p.T, t0, col0, lane);
    mma_tile(acc, s_w[0], fr[0], lane);
    mma_tile(acc, s_w[1], fr[1], lane);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const long long t = t0 + nt * 16 + (lane & 15);
      if (t < p.T) {
        const long long rowoff = t * p.Wd + col0 + in0 + (lane >> 4) * 4;
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
          float add[4] = {0.f, 0.f, 0.f, 0.f};
          if (p.dx_in != nullptr) {
            const u32x2 d = *reinterpret_cast<const u32x2*>(p.dx_in + rowoff + mt * 16);
            add[0] = bf(static_cast<uint16_t>(d[0] & 0xFFFFu));
            add[1] = bf(static_cast<uint16_t>(d[0] >> 16));
            add[2] = bf(static_cast<uint16_t>(d[1] & 0xFFFFu));
            add[3] = bf(static_cast<uint16_t>(d[1] >> 16));
          }
          u32x2 v;
          v[0] = pack2(acc[mt][nt][0] + add[0], acc[mt][nt][1] + add[1]);
          v[1] = pack2(acc[mt][nt][2] + add[2], acc[mt][nt][3] + add[3]);
          *reinterpret_cast<u32x2*>(p.dx_out + rowoff + mt * 16) = v;
        }
      }
    }
  }
}

struct ProjDwArgs {
  const uint16_t* x;
  const uint16_t* dg[2];
  float* part_w;     // [splits][nb][2][256][256]
  float* part_b;     // [splits][nb][2][256]
  long long T;
  long long per;     // tokens per split (multiple of kSlab)
  int Wd;
  int nb;
};

// One 32-token x 256-column slab of a [T, ld] matrix, as held in registers
// between its global loads and its transposed LDS store: token pairs
// (tid/32) and (tid/32)+8, column chunk tid%32 (8 columns).
struct Slab {
  u32x4 r[2][2];
};

__device__ __forceinline__ void load_slab(Slab& sl, const uint16_t* m, long long ld, long long T, long long tend,
                                          long long t0, int col0, int tid) {
  const int chunk = tid & 31;
#pragma unroll
  for (int rep = 0; rep < 2; ++rep) {
    const long long ta = t0 + 2 * ((tid >> 5) + rep * 8);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const long long t = ta + q;
      sl.r[rep][q] = (t < tend && t < T) ? load16(m + t * ld + col0 + chunk * 8) : u32x4{0u, 0u, 0u, 0u};
    }
  }
}

// Stores a slab transposed, dst[column][token]; adds its values to colsum
// (the 8 columns of this thread's chunk) when asked.
__device__ __forceinline__ void store_slab_T(uint16_t (*dst)[kSlabPad], const Slab& sl, int tid, float* colsum) {
  const int chunk = tid & 31;
#pragma unroll
  for (int rep = 0; rep < 2; ++rep) {
    const int pair = (tid >> 5) + rep * 8;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t lo = (sl.r[rep][0][j >> 1] >> ((j & 1) * 16)) & 0xFFFFu;
      const uint32_t hi = (sl.r[rep][1][j >> 1] >> ((j & 1) * 16)) & 0xFFFFu;
      *reinterpret_cast<uint32_t*>(&dst[chunk * 8 + j][2 * pair]) = lo | (hi << 16);
      if (colsum != nullptr) colsum[j] += bf(static_cast<uint16_t>(lo)) + bf(static_cast<uint16_t>(hi));
    }
  }
}

__global__ __launch_bounds__(256) void proj_dw_kernel(ProjDwArgs p) {
  __shared__ __attribute__((aligned(16))) uint16_t s_x[2][kBS][kSlabPad];   // [buf][in][token]
  __shared__ __attribute__((aligned(16))) uint16_t s_g[2][kBS][kSlabPad];   // [buf][out][token]
  __shared__ float s_cs[8][kBS];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int split = blockIdx.x;
  const int kb = blockIdx.y >> 1;
  const int g = blockIdx.y & 1;
  const int col0 = kb * kBS;
  const long long tbeg = static_cast<long long>(split) * p.per;
  const long long tend = tbeg + p.per < p.T ? tbeg + p.per : p.T;
  const uint16_t* dg = p.dg[g];

  f32x4 acc[4][16];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
    for (int nt = 0; nt < 16; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float colsum[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};

  const int n_steps = tend > tbeg ? static_cast<int>((tend - tbeg + kSlab - 1) / kSlab) : 0;
  Slab sx, sg;
  if (n_steps > 0) {
    load_slab(sx, p.x, p.Wd, p.T, tend, tbeg, col0, tid);
    load_slab(sg, dg, p.Wd, p.T, tend, tbeg, col0, tid);
    store_slab_T(s_x[0], sx, tid, nullptr);
    store_slab_T(s_g[0], sg, tid, colsum);
  }
  __syncthreads();
  for (int step = 0; step < n_steps; ++step) {
    const int buf = step & 1;
    const bool more = step + 1 < n_steps;
    if (more) {
      const long long tn = tbeg + static_cast<long long>(step + 1) * kSlab;
      load_slab(sx, p.x, p.Wd, p.T, tend, tn, col0, tid);
      load_slab(sg, dg, p.Wd, p.T, tend, tn, col0, tid);
    }
    bf16x8 a[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      a[mt] = as_bf16x8(*reinterpret_cast<const u32x4*>(&s_x[buf][wave * 64 + mt * 16 + (lane & 15)][(lane >> 4) * 8]));
    }
#pragma unroll
    for (int nt = 0; nt < 16; ++nt) {
      const bf16x8 b = as_bf16x8(*reinterpret_cast<const u32x4*>(&s_g[buf][nt * 16 + (lane & 15)][(lane >> 4) * 8]));
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) acc[mt][nt] = mfma(a[mt], b, acc[mt][nt]);
    }
    if (more) {
      store_slab_T(s_x[buf ^ 1], sx, tid, nullptr);
      store_slab_T(s_g[buf ^ 1], sg, tid, colsum);
    }
    __syncthreads();
  }

  // partial dW: rows (in) wave*64 + mt*16 + (lane/16)*4 + i, column (out) nt*16 + lane%16
  float* pw = p.part_w + ((static_cast<long long>(split) * p.nb + kb) * 2 + g) * kBS * kBS;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
    for (int nt = 0; nt < 16; ++nt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int in = wave * 64 + mt * 16 + (lane >> 4) * 4 + i;
        pw[in * kBS + nt * 16 + (lane & 15)] = acc[mt][nt][i];
      }
    }
  }
  // partial column sums of the gate gradient: fixed-order reduction over the 8 thread groups
#pragma unroll
  for (int j = 0; j < 8; ++j) s_cs[tid >> 5][(tid & 31) * 8 + j] = colsum[j];
  __syncthreads();
  {
    float s = 0.f;
    for (int r = 0; r < 8; ++r) s += s_cs[r][tid];
    p.part_b[((static_cast<long long>(split) * p.nb + kb) * 2 + g) * kBS + tid] = s;
  }
}

// dw_g[kb] = sum over splits (in order) of the partials; db likewise.
__global__ __launch_bounds__(256) void proj_dw_reduce_kernel(const float* part_w, const float* part_b, float* dw_x,
                                                             float* dw_a, float* db_x, float* db_a, int nb,
                                                             int splits) {
  const long long per_gate = static_cast<long long>(nb) * kBS * kBS;
  const long long idx = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;   // over 2 * nb * 256 * 256 (+ bias)
  const long long n_w = 2 * per_gate;
  if (idx < n_w) {
    const int g = static_cast<int>(idx / per_gate);
    const long long r = idx - g * per_gate;          // kb*65536 + in*256 + out
    const long long kb = r / (kBS * kBS);
    const long long e = r - kb * kBS * kBS;
    float s = 0.f;
    for (int sp = 0; sp < splits; ++sp) s += part_w[((static_cast<long long>(sp) * nb + kb) * 2 + g) * kBS * kBS + e];
    (g == 0 ? dw_x : dw_a)[r] = s;
    return;
  }
  const long long bi = idx - n_w;
  if (bi < 2LL * nb * kBS) {
    const int g = static_cast<int>(bi / (static_cast<long long>(nb) * kBS));
    const long long r = bi - g * static_cast<long long>(nb) * kBS;     // kb*256 + out
    const long long kb = r / kBS;
    const long long e = r - kb * kBS;
    float* dst = g == 0 ? db_x : db_a;
    if (dst == nullptr) return;
    float s = 0.f;
    for (int sp = 0; sp < splits; ++sp) s += part_b[((static_cast<long long>(sp) * nb + kb) * 2 + g) * kBS + e];
    dst[r] = s;
  }
}

int token_splits(long long T, int nb) {
  const long long tiles = (T + kTileT - 1) / kTileT;
  long long s = (256 * 2 + 2 * nb - 1) / (2 * nb);   // about two waves of workgroups over 256 CUs
  if (s < 1) s = 1;
  if (s > tiles) s = tiles;
  return static_cast<int>(s);
}

int dw_splits(long long T, int nb) {
  const long long slabs = (T + kSlab - 1) / kSlab;
  long long s = (256 + 2 * nb - 1) / (2 * nb);
  if (s < 1) s = 1;
  if (s > slabs) s = slabs;
  return static_cast<int>(s);
}

rglru_status_t check_proj(int64_t tokens, int64_t width, int64_t block) {
  if (tokens < 1 || width < 1 || block < 1) return RGLRU_ERR_INVALID_ARGUMENT;
  if (width % block != 0) return RGLRU_ERR_INVALID_ARGUMENT;
  if (block != kBS) return RGLRU_ERR_UNSUPPORTED;
  if (width > (1LL << 24) || tokens > (1LL << 40)) return RGLRU_ERR_INVALID_ARGUMENT;
  return RGLRU_OK;
}

bool al16(const void* p) { return p == nullptr || aligned_to(p, 16); }
bool al2(const void* p) { return p == nullptr || aligned_to(p, 2); }
bool al4(const void* p) { return p == nullptr || aligned_to(p, 4); }

size_t dw_ws_bytes(int64_t tokens, int64_t width) {
  const int nb = static_cast<int>(width / kBS);
  const int s = dw_splits(tokens, nb);
  return round_up(static_cast<size_t>(s) * nb * 2 * kBS * kBS * sizeof(float), 256) +
         round_up(static_cast<size_t>(s) * nb * 2 * kBS * sizeof(float), 256);
}

}  // namespace
}  // namespace rglru

using namespace rglru;

extern "C" {

size_t rglru_blockdiag_gate_proj_bwd_workspace_bytes(int64_t tokens, int64_t width, int64_t block) {
  if (check_proj(tokens, width, block) != RGLRU_OK) return 0;
  return dw_ws_bytes(tokens, width);
}

rglru_status_t rglru_blockdiag_gate_proj_fwd(int64_t tokens, int64_t width, int64_t block, const void* x,
                                             const void* w_x, const void* b_x, const void* w_a, const void* b_a,
                                             void* gate_x, void* gate_a, void* stream) {
  const rglru_status_t st0 = check_proj(tokens, width, block);
  if (st0 != RGLRU_OK) return st0;
  if (!x || !w_x || !w_a || !gate_x || !gate_a) return RGLRU_ERR_INVALID_ARGUMENT;
  if (!al16(x) || !al16(w_x) || !al16(w_a) || !al16(gate_x) || !al16(gate_a) || !al2(b_x) || !al2(b_a)) {
    return RGLRU_ERR_MISALIGNED;
  }
  const int nb = static_cast<int>(width / block);
  ProjFwdArgs a;
  a.x = static_cast<const uint16_t*>(x);
  a.w[0] = static_cast<const uint16_t*>(w_x);
  a.w[1] = static_cast<const uint16_t*>(w_a);
  a.bias[0] = static_cast<const uint16_t*>(b_x);
  a.bias[1] = static_cast<const uint16_t*>(b_a);
  a.out[0] = static_cast<uint16_t*>(gate_x);
  a.out[1] = static_cast<uint16_t*>(gate_a);
  a.T = tokens;
  a.Wd = static_cast<int>(width);
  a.splits = token_splits(tokens, nb);
  hipLaunchKernelGGL(proj_fwd_kernel, dim3(a.splits, nb * 2), dim3(256), 0, static_cast<hipStream_t>(stream), a);
  return launch_status();
}

rglru_status_t rglru_blockdiag_gate_proj_bwd(int64_t tokens, int64_t width, int64_t block, const void* x,
                                             const void* w_x, const void* w_a, const void* dgate_x,
                                             const void* dgate_a, const void* dx_in, void* dx_out, float* dw_x,
                                             float* db_x, float* dw_a, float* db_a, void* workspace,
                                             size_t workspace_bytes, void* stream) {
  const rglru_status_t st0 = check_proj(tokens, width, block);
  if (st0 != RGLRU_OK) return st0;
  if (!x || !w_x || !w_a || !dgate_x || !dgate_a || !dx_out || !dw_x || !dw_a || !workspace) {
    return RGLRU_ERR_INVALID_ARGUMENT;
  }
  if (!al16(x) || !al16(w_x) || !al16(w_a) || !al16(dgate_x) || !al16(dgate_a) || !al16(dx_in) ||
      !al16(dx_out) || !al4(dw_x) || !al4(dw_a) || !al4(db_x) || !al4(db_a) || !aligned_to(workspace, 256)) {
    return RGLRU_ERR_MISALIGNED;
  }
  if (workspace_bytes < dw_ws_bytes(tokens, width)) return RGLRU_ERR_WORKSPACE_TOO_SMALL;
  const int nb = static_cast<int>(width / block);
  hipStream_t st = static_cast<hipStream_t>(stream);

  // weight and bias gradients first: they read x and the gate gradients, and
  // dx_out may overwrite dx_in but never x
  ProjDwArgs w;
  w.x = static_cast<const uint16_t*>(x);
  w.dg[0] = static_cast<const uint16_t*>(dgate_x);
  w.dg[1] = static_cast<const uint16_t*>(dgate_a);
  const int sw = dw_splits(tokens, nb);
  const long long slabs = (tokens + kSlab - 1) / kSlab;
  w.per = ((slabs + sw - 1) / sw) * kSlab;
  w.part_w = static_cast<float*>(workspace);
  w.part_b = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                      round_up(static_cast<size_t>(sw) * nb * 2 * kBS * kBS * sizeof(float), 256));
  w.T = tokens;
  w.Wd = static_cast<int>(width);
  w.nb = nb;
  hipLaunchKernelGGL(proj_dw_kernel, dim3(sw, nb * 2), dim3(256), 0, st, w);
  rglru_status_t s1 = launch_status();
  if (s1 != RGLRU_OK) return s1;
  const long long n_red = 2LL * nb * kBS * kBS + 2LL * nb * kBS;
  hipLaunchKernelGGL(proj_dw_reduce_kernel, dim3(static_cast<unsigned>((n_red + 255) / 256)), dim3(256), 0, st,
                     static_cast<const float*>(w.part_w), static_cast<const float*>(w.part_b), dw_x, dw_a, db_x,
                     db_a, nb, sw);
  s1 = launch_status();
  if (s1 != RGLRU_OK) return s1;

  ProjDxArgs d;
  d.w[0] = static_cast<const uint16_t*>(w_x);
  d.w[1] = static_cast<const uint16_t*>(w_a);
  d.dg[0] = static_cast<const uint16_t*>(dgate_x);
  d.dg[1] = static_cast<const uint16_t*>(dgate_a);
  d.dx_in = static_cast<const uint16_t*>(dx_in);
  d.dx_out = static_cast<uint16_t*>(dx_out);
  d.T = tokens;
  d.Wd = static_cast<int>(width);
  d.splits = token_splits(tokens, nb);
  hipLaunchKernelGGL(proj_dx_kernel, dim3(d.splits, nb * 2), dim3(256), 0, st, d);
  return launch_status();
}

}  // extern "C"
