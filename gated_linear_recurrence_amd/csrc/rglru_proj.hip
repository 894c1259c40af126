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
// gradient stream into a ring of LDS buffers (global_load_lds) and the MFMA
// operands come out with the gfx950 transpose read; each workgroup owns one
// (block, gate) and a contiguous token range, keeps the whole 256x256 float32
// block in accumulators, and writes a partial that a second kernel sums over
// token ranges in a fixed order (deterministic).
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

// ---------------------------------------------------------------- weight gradient
//
// dw_g[kb] = x[:, kb]^T @ dgate_g[:, kb]: the contraction runs over tokens,
// which are strided in memory for both operands. A workgroup of 8 waves owns
// one (block, gate) and a contiguous token range; the 256x256 float32 block
// lives in accumulators, wave w holding input rows 64*(w%4) .. +63 and output
// columns 128*(w/4) .. +127 (128 per lane; both gates at once would take the
// whole register file). Slabs of 32 tokens of x and of the gate gradient
// (16 KiB each, token-major as in memory) stream into a ring of LDS buffers
// with global_load_lds, kDwBufs - 1 steps ahead; the MFMA operands (8
// consecutive tokens of one column per lane) come out of LDS with the gfx950
// transpose read ds_read_b64_tr_b16. Rows are stored with their 32-byte
// chunks permuted (chunk c of token row r at position c ^ (r % 16)) so that
// the rows one transpose read touches fall on different banks. The two gates
// of one (block, range) run on the same XCD at the same time, so the second
// read of x is served by that XCD's L2. The partial of the range is written
// in the accumulators' own layout (16 contiguous bytes per lane) and
// proj_dw_reduce_kernel sums the partials of all ranges in a fixed order.

constexpr int kKT = 32;               // tokens per step
constexpr int kDwBufs = 4;            // LDS ring depth (32 KiB per step)
constexpr int kDwWaves = 8;
constexpr int kDwIns = 4;             // 1 KiB loads per wave per step (32 KiB / 8 waves)

// 16 bytes per lane from global memory straight into LDS (lane l writes
// dst + 16 * l). The 16-byte form exists only on gfx950, so the host pass does
// not see it.
__device__ __forceinline__ void lds_dma16(const void* src, void* dst) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
#endif
}

// waits until at most N of this wave's global loads and none of its LDS
// accesses are outstanding (gfx9 s_waitcnt layout: vmcnt[3:0], expcnt[6:4],
// lgkmcnt[11:8])
template <int N>
__device__ __forceinline__ void wait_vm_lds() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0070 | N);
}

// Transpose read ds_read_b64_tr_b16 at LDS byte address `addr`: in each group
// of 16 lanes, lane i receives element (i & 3) of the 8 bytes addressed by
// lanes (i >> 2) + 4m, m = 0..3. Issued as inline assembly: the compiler
// would otherwise make every such read wait for all LDS-bound global loads in
// flight (it cannot tell which ring buffer they land in). Completion is
// waited for explicitly with lds_wait.
__device__ __forceinline__ u32x2 lds_read_tr(uint32_t addr) {
  u32x2 d;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(d) : "v"(addr));
  return d;
}

// waits until at most N LDS reads are outstanding; the operands tie the
// values read so that no use moves above the wait
template <int N>
__device__ __forceinline__ void lds_wait(u32x2& x, u32x2& y) {
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(x), "+v"(y) : "n"(N));
}

struct ProjDwArgs {
  const uint16_t* x;
  const uint16_t* dg[2];
  float* part_w;   // [split][block][gate][16 m-tiles][16 n-tiles][64 lanes][4]
  float* part_b;   // [split][block][gate][256]
  long long T;
  long long per;   // tokens per split (a multiple of kKT)
  int Wd;
  int nb;
  int splits;
};

// LDS byte offsets, within one slab, of the two transpose reads that give a
// lane its MFMA operand for columns col0 .. col0+15 (lane l: column
// col0 + l % 16, tokens (l / 16) * 8 .. +7). Source lane s of each 16-lane
// group addresses token row (s / 4) (+4 for the second read) at columns
// col0 + 4 * (s % 4) .. +3; row r stores 32-byte chunk c at position
// c ^ (r % 16).
__device__ __forceinline__ uint32_t frag_off(int col0, int lane, int half) {
  const int g = lane >> 4;
  const int sl = lane & 15;
  const int r = g * 8 + (sl >> 2) + half * 4;
  const int chunk = col0 >> 4;
  return static_cast<uint32_t>(r * (kBS * 2) + ((chunk ^ (r & 15)) << 5) + (sl & 3) * 8);
}

__device__ __forceinline__ bf16x8 frag_of(u32x2 lo, u32x2 hi) {
  return as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
}

__global__ __launch_bounds__(kDwWaves * 64) void proj_dw_kernel(ProjDwArgs p) {
  __shared__ __attribute__((aligned(16))) uint16_t s_slab[kDwBufs][2][kKT][kBS];   // [buf][x, dgate][token][col]
  __shared__ float s_cs[4][kBS];
  constexpr uint32_t kSlabBytes = kKT * kBS * 2;
  // workgroup id -> (gate, range, block): ids 8 apart run on the same XCD, so
  // the two gates of one (range, block) are paired that way
  const int id = blockIdx.x;
  const int gate = (id >> 3) & 1;
  const int pair = (id >> 4) * 8 + (id & 7);
  if (pair >= p.splits * p.nb) return;
  const int split = pair / p.nb;
  const int kb = pair - split * p.nb;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ib = wave & 3;             // input rows ib*64 .. +63
  const int jb = wave >> 2;            // output columns jb*128 .. +127
  const long long tbeg = static_cast<long long>(split) * p.per;
  const long long tend = tbeg + p.per < p.T ? tbeg + p.per : p.T;
  const int n_steps = tend > tbeg ? static_cast<int>((tend - tbeg + kKT - 1) / kKT) : 0;

  // this lane's part of the step loads: kDwIns instructions of 1 KiB, each 2
  // token rows of one tensor (32 lanes per row); instruction ins = wave *
  // kDwIns + u covers tensor ins / 16 (x, then the gate gradient), rows
  // 2 * (ins % 16) and the next. Byte offsets from the step's first token.
  const uint16_t* base_x = p.x + kb * kBS;
  const uint16_t* base_g = p.dg[gate] + kb * kBS;
  uint32_t voff[kDwIns];
  int row[kDwIns];
#pragma unroll
  for (int u = 0; u < kDwIns; ++u) {
    const int ins = wave * kDwIns + u;
    const int r = (ins & 15) * 2 + (lane >> 5);
    const int pos = lane & 31;           // 16-byte granule position in the LDS row
    const int gran = (((pos >> 1) ^ (r & 15)) << 1) | (pos & 1);
    voff[u] = static_cast<uint32_t>(r) * static_cast<uint32_t>(p.Wd) * 2u + gran * 16u;
    row[u] = r;
  }
  // loads of step `st`; in the range's last step, rows past its end are
  // zero-filled instead (LDS stores, waited for with the loads)
  auto issue = [=](int st) {
    const long long t0 = tbeg + static_cast<long long>(st) * kKT;
    const int valid = tend - t0 < kKT ? static_cast<int>(tend - t0) : kKT;
#pragma unroll
    for (int u = 0; u < kDwIns; ++u) {
      const int ins = wave * kDwIns + u;
      const char* sb = reinterpret_cast<const char*>(((ins >> 4) == 0 ? base_x : base_g) + t0 * p.Wd);
      uint16_t* dst = &s_slab[st % kDwBufs][ins >> 4][(ins & 15) * 2][0];
      if (valid == kKT || row[u] < valid) {
        lds_dma16(sb + voff[u], dst);
      } else {
        *reinterpret_cast<u32x4*>(dst + lane * 8) = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };

  // LDS byte addresses of this lane's operand reads in ring buffer 0
  typedef __attribute__((address_space(3))) uint16_t lds_u16;
  const uint32_t ring0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_u16*)(&s_slab[0][0][0][0])));
  uint32_t a_off[4][2];
  uint32_t b_off[8][2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) a_off[mt][h] = ring0 + frag_off(ib * 64 + mt * 16, lane, h);
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) b_off[nt][h] = ring0 + kSlabBytes + frag_off(jb * 128 + nt * 16, lane, h);
  }

  f32x4 acc[4][8];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float colsum[2] = {0.f, 0.f};        // output columns jb*128 + (2*ib + i)*16 + lane%16

#pragma unroll
  for (int d = 0; d < kDwBufs - 1; ++d) {
    if (d < n_steps) issue(d);
  }
  for (int st = 0; st < n_steps; ++st) {
    static_assert(kDwBufs == 4, "the wait ladder below assumes 3 steps in flight");
    const int ahead = n_steps - 1 - st;
    if (ahead >= 2) {
      wait_vm_lds<2 * kDwIns>();
    } else if (ahead == 1) {
      wait_vm_lds<kDwIns>();
    } else {
      wait_vm_lds<0>();
    }
    // every wave's loads of this step are in LDS, and every wave is done
    // reading the buffer the next issue overwrites (read in step st - 1)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (ahead >= 3) issue(st + 3);
    const uint32_t bo = static_cast<uint32_t>(st % kDwBufs) * (2 * kSlabBytes);
    // at most 14 reads in flight (the LDS counter holds 15): the 4 row
    // operands and the next 3 column operands
    u32x2 ra[4][2];
    u32x2 rb[8][2];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      ra[mt][0] = lds_read_tr(a_off[mt][0] + bo);
      ra[mt][1] = lds_read_tr(a_off[mt][1] + bo);
    }
#pragma unroll
    for (int nt = 0; nt < 3; ++nt) {
      rb[nt][0] = lds_read_tr(b_off[nt][0] + bo);
      rb[nt][1] = lds_read_tr(b_off[nt][1] + bo);
    }
    lds_wait<6>(ra[0][0], ra[0][1]);
    lds_wait<6>(ra[1][0], ra[1][1]);
    lds_wait<6>(ra[2][0], ra[2][1]);
    lds_wait<6>(ra[3][0], ra[3][1]);
    bf16x8 a[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) a[mt] = frag_of(ra[mt][0], ra[mt][1]);
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      // reads complete in order; in flight now: column operands nt .. min(nt + 2, 7)
      if (nt < 6) {
        lds_wait<4>(rb[nt][0], rb[nt][1]);
      } else if (nt == 6) {
        lds_wait<2>(rb[nt][0], rb[nt][1]);
      } else {
        lds_wait<0>(rb[nt][0], rb[nt][1]);
      }
      if (nt + 3 < 8) {
        rb[nt + 3][0] = lds_read_tr(b_off[nt + 3][0] + bo);
        rb[nt + 3][1] = lds_read_tr(b_off[nt + 3][1] + bo);
      }
      const bf16x8 b = frag_of(rb[nt][0], rb[nt][1]);
      if ((nt >> 1) == ib) {
        float cs = 0.f;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const uint32_t w = rb[nt][h][e];
            cs += __uint_as_float(w << 16) + __uint_as_float(w & 0xFFFF0000u);
          }
        }
        colsum[nt & 1] += cs;
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) acc[mt][nt] = mfma(a[mt], b, acc[mt][nt]);
    }
    asm volatile("" ::: "memory");
  }

  // partial in the accumulators' own layout: tile (m, n) of 16x16, lane, 4 floats
  float* pw = p.part_w + ((static_cast<long long>(split) * p.nb + kb) * 2 + gate) * (kBS * kBS);
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const long long tile = (ib * 4 + mt) * 16 + jb * 8 + nt;
      *reinterpret_cast<f32x4*>(pw + (tile * 64 + lane) * 4) = acc[mt][nt];
    }
  }
  // column sums of the gate gradient: the 4 lane groups hold different
  // tokens of the same columns; fixed-order sum through LDS
#pragma unroll
  for (int i = 0; i < 2; ++i) s_cs[lane >> 4][jb * 128 + (2 * ib + i) * 16 + (lane & 15)] = colsum[i];
  __syncthreads();
  if (threadIdx.x < kBS) {
    const int c = threadIdx.x;
    const float sum = ((s_cs[0][c] + s_cs[1][c]) + s_cs[2][c]) + s_cs[3][c];
    p.part_b[((static_cast<long long>(split) * p.nb + kb) * 2 + gate) * kBS + c] = sum;
  }
}

// dw_g[kb] and db_g[kb]: fixed-order sums over the token ranges. Thread =
// (gate, block, tile, lane) of the partial layout; it writes 4 floats of dw
// (rows tile_m*16 + (lane/16)*4 .. +3, column tile_n*16 + lane%16).
__global__ __launch_bounds__(256) void proj_dw_reduce_kernel(const float* part_w, const float* part_b, float* dw_x,
                                                             float* dw_a, float* db_x, float* db_a, int nb,
                                                             int splits) {
  const long long n_groups = 2LL * nb * 256 * 64;   // (gate, block) x 256 tiles x 64 lanes
  const long long idx = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  if (idx < n_groups) {
    const long long gk = idx / (256 * 64);          // (block, gate) pair: kb * 2 + g
    const int rem = static_cast<int>(idx - gk * 256 * 64);
    const int tile = rem >> 6;
    const int lane = rem & 63;
    const int kb = static_cast<int>(gk >> 1);
    const int g = static_cast<int>(gk & 1);
    f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int sp = 0; sp < splits; ++sp) {
      const float* src = part_w + ((static_cast<long long>(sp) * nb + kb) * 2 + g) * (kBS * kBS) +
                         (static_cast<long long>(tile) * 64 + lane) * 4;
      s += *reinterpret_cast<const f32x4*>(src);
    }
    const int in0 = (tile >> 4) * 16 + (lane >> 4) * 4;
    const int out = (tile & 15) * 16 + (lane & 15);
    float* dw = (g == 0 ? dw_x : dw_a) + static_cast<long long>(kb) * kBS * kBS;
#pragma unroll
    for (int i = 0; i < 4; ++i) dw[(in0 + i) * kBS + out] = s[i];
    return;
  }
  const long long bi = idx - n_groups;
  if (bi < 2LL * nb * kBS) {
    const int g = static_cast<int>(bi / (static_cast<long long>(nb) * kBS));
    const long long r = bi - g * static_cast<long long>(nb) * kBS;     // kb*256 + out
    const long long kb = r / kBS;
    const long long e = r - kb * kBS;
    float* dst = g == 0 ? db_x : db_a;
    if (dst == nullptr) return;
    float sum = 0.f;
    for (int sp = 0; sp < splits; ++sp) sum += part_b[((static_cast<long long>(sp) * nb + kb) * 2 + g) * kBS + e];
    dst[r] = sum;
  }
}

int token_splits(long long T, int nb) {
  const long long tiles = (T + kTileT - 1) / kTileT;
  long long s = (256 * 2 + 2 * nb - 1) / (2 * nb);   // about two waves of workgroups over 256 CUs
  if (s < 1) s = 1;
  if (s > tiles) s = tiles;
  return static_cast<int>(s);
}

// token ranges of the weight-gradient kernel: about one workgroup per CU
// (each holds a whole CU's worth of registers), no empty range
int dw_splits(long long T, int nb) {
  const long long steps = (T + kKT - 1) / kKT;
  long long s = 256 / (2 * nb);
  if (s < 1) s = 1;
  if (s > steps) s = steps;
  const long long per = (steps + s - 1) / s;
  return static_cast<int>((steps + per - 1) / per);
}

long long dw_per(long long T, int splits) {
  const long long steps = (T + kKT - 1) / kKT;
  return ((steps + splits - 1) / splits) * kKT;
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
  w.per = dw_per(tokens, sw);
  w.part_w = static_cast<float*>(workspace);
  w.part_b = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                      round_up(static_cast<size_t>(sw) * nb * 2 * kBS * kBS * sizeof(float), 256));
  w.T = tokens;
  w.Wd = static_cast<int>(width);
  w.nb = nb;
  w.splits = sw;
  const long long pairs = static_cast<long long>(sw) * nb;
  hipLaunchKernelGGL(proj_dw_kernel, dim3(static_cast<unsigned>(((pairs + 7) / 8) * 16)), dim3(kDwWaves * 64), 0,
                     st, w);
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
