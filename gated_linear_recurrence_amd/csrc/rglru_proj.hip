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
// bf16 operands, float32 accumulation: v_mfma_f32_32x32x16_bf16 in the
// forward, v_mfma_f32_16x16x32_bf16 in the backward (A 16x32, B 32x16; lane l
// holds row/column l%16 and k = (l/16)*8 .. +7; D lane l holds column l%16,
// rows (l/16)*4 .. +3).
//
// Forward and dx kernels: a workgroup of 8 waves owns one block and a
// contiguous token range. Its weight fragments (bf16, 128 VGPRs per lane) are
// loaded once; 32-token tiles of the token-major operands stream through a
// ring of LDS buffers with global_load_lds, steps ahead of the multiply, and
// the outputs leave through a per-wave LDS staging area as whole row segments.
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
constexpr int kKT = 32;           // tokens per step
constexpr int kWaves8 = 8;        // waves per workgroup of every kernel here
constexpr uint32_t kSlabBytes = kKT * kBS * 2;   // one 32-row x 256-column bf16 slab

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// v_mfma_f32_32x32x16_bf16: A 32x16, B 16x32; lane l holds row/column l%32
// and k = (l/32)*8 .. +7; D lane l holds column l%32, register r row
// (r/4)*8 + (l/32)*4 + r%4. One wave sustains about 2.4 times the rate of the
// 16x16x32 form, which needs several waves per SIMD to approach its peak.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ u32x4 load16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }

__device__ __forceinline__ uint32_t pack2(float lo, float hi) { return f32x2_to_bf16x2(lo, hi); }

__device__ __forceinline__ float bf(uint16_t v) { return bf16_bits_to_f32(v); }

// 16 bytes per lane from global memory straight into LDS (lane l writes
// dst + 16 * l). The 16-byte form exists only on gfx950, so the host pass does
// not see it.
__device__ __forceinline__ void lds_dma16(const void* src, void* dst) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
#endif
}

// waits until at most N of this wave's vector-memory operations and none of
// its LDS accesses are outstanding. gfx9 s_waitcnt layout: vmcnt[3:0] and
// [15:14], expcnt[6:4], lgkmcnt[11:8]. Vector-memory operations (loads into
// LDS and stores alike) retire in issue order on this architecture.
template <int N>
__device__ __forceinline__ void wait_vm_lds() {
  static_assert(N >= 0 && N < 64, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | 0x0070);
}

// wait_vm_lds<ns * S + nd * D>() for runtime ns <= NS, nd <= ND: a step
// issues D loads and S stores per wave, and the loads of the step about to be
// read are followed by ns steps of stores and nd steps of loads
template <int S, int D, int NS, int ND>
__device__ __forceinline__ void wait_ring_nd(int nd) {
  if constexpr (ND > 0) {
    if (nd == ND) {
      wait_vm_lds<NS * S + ND * D>();
      return;
    }
    wait_ring_nd<S, D, NS, ND - 1>(nd);
  } else {
    wait_vm_lds<NS * S>();
  }
}

template <int S, int D, int NS, int ND>
__device__ __forceinline__ void wait_ring(int ns, int nd) {
  if constexpr (NS > 0) {
    if (ns == NS) {
      wait_ring_nd<S, D, NS, ND>(nd);
      return;
    }
    wait_ring<S, D, NS - 1, ND>(ns, nd);
  } else {
    wait_ring_nd<S, D, 0, ND>(nd);
  }
}

// LDS reads issued as inline assembly: the compiler would otherwise make each
// of them wait for every LDS-bound global load in flight (it cannot tell
// which ring buffer those land in). Completion is waited for with lds_wait,
// whose operands tie the values read so that no use moves above the wait.
__device__ __forceinline__ u32x4 lds_read16(uint32_t addr) {
  u32x4 d;
  asm volatile("ds_read_b128 %0, %1" : "=v"(d) : "v"(addr));
  return d;
}

__device__ __forceinline__ u32x2 lds_read8(uint32_t addr) {
  u32x2 d;
  asm volatile("ds_read_b64 %0, %1" : "=v"(d) : "v"(addr));
  return d;
}

__device__ __forceinline__ void lds_write8(uint32_t addr, u32x2 v) {
  asm volatile("ds_write_b64 %0, %1" : : "v"(addr), "v"(v));
}

// Transpose read ds_read_b64_tr_b16 (gfx950): in each group of 16 lanes, lane
// i receives element (i & 3) of the 8 bytes addressed by lanes (i >> 2) + 4m,
// m = 0..3.
__device__ __forceinline__ u32x2 lds_read_tr(uint32_t addr) {
  u32x2 d;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(d) : "v"(addr));
  return d;
}

// waits until at most N LDS operations of this wave are outstanding (they
// complete in order; the counter holds at most 15)
template <int N>
__device__ __forceinline__ void lds_wait(u32x4& x, u32x4& y) {
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(x), "+v"(y) : "n"(N));
}

template <int N>
__device__ __forceinline__ void lds_wait(u32x2& x, u32x2& y) {
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(x), "+v"(y) : "n"(N));
}

template <int N>
__device__ __forceinline__ void lds_wait1(u32x4& x) {
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(x) : "n"(N));
}

__device__ __forceinline__ bf16x8 frag_of(u32x2 lo, u32x2 hi) {
  return as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  typedef __attribute__((address_space(3))) const char lds_char;
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_char*)(p)));   // generic -> LDS offset
}

// Slab layouts in LDS: 32 rows of 512 bytes; the 16-byte granules of a row
// are permuted so that the reads of one operand fall on distinct banks.
//   kSwz16: granule g of row r at position g ^ (r % 16)  (16-byte row reads:
//           16 rows at one granule, 512 bytes apart, fall on 16 distinct
//           groups of 4 banks)
//   kSwz32: 32-byte chunk c of row r at position c ^ (r % 16), granules
//           within a chunk in order                      (transpose reads)
// The map is an involution: it gives the source granule of a position too.
constexpr int kSwz16 = 0;
constexpr int kSwz32 = 1;

template <int SWZ>
__device__ __forceinline__ int swz_gran(int g, int r) {
  if constexpr (SWZ == kSwz16) {
    return g ^ (r & 15);
  } else {
    return (((g >> 1) ^ (r & 15)) << 1) | (g & 1);
  }
}

// A row of zeros in device memory: slab rows past the end of a token range
// are loaded from it, so that every load instruction of a step is issued by
// every lane (the waits count issued instructions).
__device__ __attribute__((aligned(16))) uint16_t g_zero_row[kBS];

// Piece j (rows 2j and 2j + 1, 1 KiB) of a slab whose row r is
// src + r * ld (256 bf16): one LDS-bound load of 16 bytes per lane; rows at
// or past `valid` read zeros.
template <int SWZ>
__device__ __forceinline__ void slab_piece(const uint16_t* src, long long ld, int j, int valid, uint16_t* slab,
                                           int lane) {
  const int r = 2 * j + (lane >> 5);
  const uint16_t* row = r < valid ? src + r * ld : g_zero_row;
  lds_dma16(row + swz_gran<SWZ>(lane & 31, r) * 8, slab + j * 2 * kBS);
}

// LDS byte offset, within a kSwz32 slab, of one of the two transpose reads
// that give a lane its MFMA operand for columns col0 .. col0+15 of 8
// consecutive rows (lane l: column col0 + l % 16, rows (l / 16) * 8 .. +7):
// source lane s of each 16-lane group addresses row (s / 4) (+4 for the
// second read) at columns col0 + 4 * (s % 4) .. +3.
__device__ __forceinline__ uint32_t frag_off(int col0, int lane, int half) {
  const int g = lane >> 4;
  const int sl = lane & 15;
  const int r = g * 8 + (sl >> 2) + half * 4;
  const int chunk = col0 >> 4;
  return static_cast<uint32_t>(r * (kBS * 2) + ((chunk ^ (r & 15)) << 5) + (sl & 3) * 8);
}

// The same for a 32x32x16 A operand: rows h*16 .. +15 of the slab are the
// k-step; lane l takes column col0 + l % 32, rows (l / 32) * 8 .. +7 of it, the
// two reads giving rows +0 .. 3 and +4 .. 7 (source lane s of each 16-lane
// group addresses row (s / 4) at columns 4 * (s % 4) .. +3 of its 16 columns).
__device__ __forceinline__ uint32_t frag_off32(int col0, int lane, int h, int half) {
  const int g = lane >> 4;
  const int sl = lane & 15;
  const int r = h * 16 + (g >> 1) * 8 + half * 4 + (sl >> 2);
  const int chunk = (col0 >> 4) + (g & 1);
  return static_cast<uint32_t>(r * (kBS * 2) + ((chunk ^ (r & 15)) << 5) + (sl & 3) * 8);
}

// LDS byte offset, within a kSwz16 slab, of the 16 bytes at row r, columns
// 8 * g .. +7
__device__ __forceinline__ uint32_t row_off16(int r, int g) {
  return static_cast<uint32_t>(r * (kBS * 2) + (swz_gran<kSwz16>(g, r) << 4));
}

// token range of a workgroup: [tbeg, tend) and its step count
struct Range {
  long long tbeg;
  long long tend;
  int n_steps;
};

__device__ __forceinline__ Range token_range(int idx, long long per, long long T) {
  Range r;
  r.tbeg = static_cast<long long>(idx) * per;
  r.tend = r.tbeg + per < T ? r.tbeg + per : T;
  r.n_steps = r.tend > r.tbeg ? static_cast<int>((r.tend - r.tbeg + kKT - 1) / kKT) : 0;
  return r;
}

// ---------------------------------------------------------------- forward
//
// gate_g[t, kb*256 + o] = b_g[o] + sum_i x[t, kb*256 + i] w_g[kb][i][o].
// v_mfma_f32_32x32x16_bf16 with A = w_g^T (rows o, k = i) held in registers
// and B = x^T (k = i, columns t) from the LDS ring, so that D holds, per lane,
// one token and 4 groups of 4 consecutive outputs. Wave w computes gate w / 4,
// outputs 64 * (w % 4) .. +63: 2 m-tiles of 32 outputs x 16 k-steps of 16
// inputs, accumulated from the bias in input order. The weights reach
// registers through the same LDS buffers (kSwz32 slabs of 32 input rows) and
// transpose reads.

constexpr int kFwdBufs = 4;                   // ring of x slabs (16 KiB each)
constexpr int kFwdDma = 2;                    // 1 KiB loads per wave per step
constexpr int kFwdStores = 4;                 // 16-byte stores per wave per step
constexpr int kStagePitch = 144;              // bytes per staged output row (128 + 16: conflict-free)
constexpr int kFwdAhead = 4;                  // k-steps of token operands read ahead
static_assert(kFwdAhead == 4, "the wait ladder in proj_fwd_kernel assumes 4 reads in flight");

struct ProjFwdArgs {
  const uint16_t* x;
  const uint16_t* w[2];
  const uint16_t* bias[2];
  uint16_t* out[2];
  long long T;
  long long per;   // tokens per range (a multiple of kKT)
  int Wd;
  int nb;
  int ranges;
};

__global__ __launch_bounds__(kWaves8 * 64) void proj_fwd_kernel(ProjFwdArgs p) {
  __shared__ __attribute__((aligned(16))) uint16_t s_ring[kFwdBufs][kKT][kBS];
  // per-wave output staging: 32 tokens x 64 outputs, so that each store
  // writes whole 128-byte row segments
  __shared__ __attribute__((aligned(16))) char s_stage[kWaves8][kKT][kStagePitch];
  const int id = blockIdx.x;
  const int range = id / p.nb;
  const int kb = id - range * p.nb;
  if (range >= p.ranges) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int gw = wave >> 2;                 // gate of this wave
  const int ob = (wave & 3) * 64;           // first output (within the block) of this wave
  const Range rg = token_range(range, p.per, p.T);
  const uint32_t ring0 = lds_addr(&s_ring[0][0][0]);

  // weights: 16 slabs (gate, 32 input rows = 2 k-steps) in 4 rounds of 4 ring buffers
  bf16x8 wr[2][16];                         // [m-tile][k-step]
#pragma unroll
  for (int round = 0; round < 4; ++round) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int sl = round * 4 + b;         // gate sl / 8, input rows (sl % 8) * 32 .. +31
      const uint16_t* src = p.w[sl >> 3] + static_cast<long long>(kb) * kBS * kBS + (sl & 7) * kKT * kBS;
#pragma unroll
      for (int u = 0; u < 2; ++u) slab_piece<kSwz32>(src, kBS, wave * 2 + u, kKT, &s_ring[b][0][0], lane);
    }
    wait_vm_lds<0>();
    __syncthreads();
    if (gw == (round >> 1)) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int ks = ((round & 1) * 4 + b) * 2 + h;
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) {
            u32x2 lo = lds_read_tr(ring0 + b * kSlabBytes + frag_off32(ob + mt * 32, lane, h, 0));
            u32x2 hi = lds_read_tr(ring0 + b * kSlabBytes + frag_off32(ob + mt * 32, lane, h, 1));
            lds_wait<0>(lo, hi);
            wr[mt][ks] = frag_of(lo, hi);
          }
        }
      }
    }
    __syncthreads();
  }

  // bias of this lane's outputs ob + mt*32 + 8j + (lane/32)*4 + i, as bf16
  // pairs (i = 0, 1 and 2, 3)
  uint32_t bias2[2][4][2];
  const uint16_t* bsrc = p.bias[gw];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int o = kb * kBS + ob + mt * 32 + j * 8 + (lane >> 5) * 4;
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        bias2[mt][j][k] = bsrc != nullptr ? (static_cast<uint32_t>(bsrc[o + 2 * k]) |
                                             (static_cast<uint32_t>(bsrc[o + 2 * k + 1]) << 16))
                                          : 0u;
      }
    }
  }

  // x slabs: piece wave * 2 + u of each step
  const uint16_t* xsrc = p.x + kb * kBS;
  auto issue = [=](int st) {
    const long long t0 = rg.tbeg + static_cast<long long>(st) * kKT;
    const int valid = rg.tend - t0 < kKT ? static_cast<int>(rg.tend - t0) : kKT;
#pragma unroll
    for (int u = 0; u < kFwdDma; ++u) {
      slab_piece<kSwz16>(xsrc + t0 * p.Wd, p.Wd, wave * kFwdDma + u, valid, &s_ring[st % kFwdBufs][0][0], lane);
    }
  };
  // B operand of k-step ks: row lane%32, columns ks*16 + (lane/32)*8 .. +7
  uint32_t xoff[16];
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) xoff[ks] = row_off16(lane & 31, ks * 2 + (lane >> 5));
  uint16_t* obase = p.out[gw] + kb * kBS + ob + (lane & 7) * 8;   // lane's 16 bytes of a staged row
  const uint32_t stage_w = lds_addr(&s_stage[wave][lane & 31][(lane >> 5) * 8]);
  const uint32_t stage_r = lds_addr(&s_stage[wave][lane >> 3][(lane & 7) * 16]);

#pragma unroll
  for (int d = 0; d < kFwdBufs - 1; ++d) {
    if (d < rg.n_steps) issue(d);
  }
  for (int st = 0; st < rg.n_steps; ++st) {
    const int ahead = rg.n_steps - 1 - st;
    wait_ring<kFwdStores, kFwdDma, kFwdBufs - 1, kFwdBufs - 2>(st < kFwdBufs - 1 ? st : kFwdBufs - 1,
                                                              ahead < kFwdBufs - 2 ? ahead : kFwdBufs - 2);
    // every wave's loads of this step are in LDS, and every wave is done
    // reading the buffer the next issue overwrites (read in step st - 1)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (ahead >= kFwdBufs - 1) issue(st + kFwdBufs - 1);
    const uint32_t sb = ring0 + static_cast<uint32_t>(st % kFwdBufs) * kSlabBytes;
    f32x16 acc[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          acc[mt][j * 4 + 2 * k] = __uint_as_float(bias2[mt][j][k] << 16);
          acc[mt][j * 4 + 2 * k + 1] = __uint_as_float(bias2[mt][j][k] & 0xFFFF0000u);
        }
      }
    }
    // token operands, kFwdAhead k-steps in flight
    u32x4 xb[16];
#pragma unroll
    for (int ks = 0; ks < kFwdAhead; ++ks) xb[ks] = lds_read16(sb + xoff[ks]);
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      // in flight: k-steps ks .. min(ks + kFwdAhead - 1, 15)
      if (ks <= 16 - kFwdAhead) {
        lds_wait1<kFwdAhead - 1>(xb[ks]);
      } else if (ks == 17 - kFwdAhead) {
        lds_wait1<kFwdAhead - 2>(xb[ks]);
      } else if (ks == 18 - kFwdAhead) {
        lds_wait1<kFwdAhead - 3>(xb[ks]);
      } else {
        lds_wait1<0>(xb[ks]);
      }
      if (ks + kFwdAhead < 16) xb[ks + kFwdAhead] = lds_read16(sb + xoff[ks + kFwdAhead]);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) acc[mt] = mfma32(wr[mt][ks], as_bf16x8(xb[ks]), acc[mt]);
    }
    asm volatile("" ::: "memory");
    // D lane l: token l%32, outputs mt*32 + 8j + (l/32)*4 .. +3 -> staging
    // (LDS accesses of one wave complete in order)
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x2 v;
        v[0] = pack2(acc[mt][j * 4 + 0], acc[mt][j * 4 + 1]);
        v[1] = pack2(acc[mt][j * 4 + 2], acc[mt][j * 4 + 3]);
        lds_write8(stage_w + mt * 64 + j * 16, v);
      }
    }
    // staged rows -> global: lane l stores bytes 16 * (l % 8) .. +15 of rows
    // l / 8 + 8 * q
    u32x4 sv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) sv[q] = lds_read16(stage_r + q * 8 * kStagePitch);
    lds_wait<0>(sv[0], sv[1]);
    lds_wait<0>(sv[2], sv[3]);
    const long long t0 = rg.tbeg + static_cast<long long>(st) * kKT;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const long long t = t0 + q * 8 + (lane >> 3);
      if (ahead > 0 || t < rg.tend) *reinterpret_cast<u32x4*>(obase + t * p.Wd) = sv[q];
    }
    // the stores are issued before the next step's wait counts them
    asm volatile("" ::: "memory");
  }
}

// ---------------------------------------------------------------- dx
//
// dx[t, kb*256 + i] = dx_in[t, kb*256 + i]
//                     + sum_g sum_o dgate_g[t, kb*256 + o] w_g[kb][i][o].
// MFMA with A = w_g (rows i, k = o: contiguous in memory, loaded straight
// into registers) and B = dgate_g^T (k = o, columns t) from the LDS ring; D
// holds 4 consecutive dx channels of one token per lane. Wave w computes
// inputs 32 * w .. +31 (2 m-tiles) over K = 512 (both gates, 16 k-steps).
// dx_in, when given, rides in the ring as a third slab and initialises the
// accumulators.

constexpr int kDxBufs = 3;       // ring of (dgate_x, dgate_a[, dx_in]) slab groups
constexpr int kDxStores = 4;     // 8-byte stores per wave per step (2 token tiles x 2 m-tiles)

struct ProjDxArgs {
  const uint16_t* w[2];
  const uint16_t* dg[2];
  const uint16_t* dx_in;
  uint16_t* dx_out;
  long long T;
  long long per;   // tokens per range (a multiple of kKT)
  int Wd;
  int nb;
  int ranges;
};

template <bool RES>
__global__ __launch_bounds__(kWaves8 * 64) void proj_dx_kernel(ProjDxArgs p) {
  constexpr int kQ = RES ? 3 : 2;                 // slabs per step
  constexpr int kDma = kQ * 16 / kWaves8;         // 1 KiB loads per wave per step
  __shared__ __attribute__((aligned(16))) uint16_t s_ring[kDxBufs][kQ][kKT][kBS];
  const int id = blockIdx.x;
  const int range = id / p.nb;
  const int kb = id - range * p.nb;
  if (range >= p.ranges) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ib = wave * 32;                       // first input channel (within the block) of this wave
  const Range rg = token_range(range, p.per, p.T);
  const uint32_t ring0 = lds_addr(&s_ring[0][0][0][0]);

  // weights: lane l holds w_g[kb][ib + mt*16 + l%16][(ks%8)*32 + (l/16)*8 .. +7], g = ks / 8
  bf16x8 wr[2][16];
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) {
    const uint16_t* wb = p.w[ks >> 3] + static_cast<long long>(kb) * kBS * kBS + (ks & 7) * 32 + (lane >> 4) * 8;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) wr[mt][ks] = as_bf16x8(load16(wb + (ib + mt * 16 + (lane & 15)) * kBS));
  }

  // loads of step st: pieces 2 * wave and 2 * wave + 1 of each slab
  const uint16_t* src0 = p.dg[0] + kb * kBS;
  const uint16_t* src1 = p.dg[1] + kb * kBS;
  const uint16_t* src2 = RES ? p.dx_in + kb * kBS : nullptr;
  const int Wd = p.Wd;
  auto issue = [=](int st) {
    const long long t0 = rg.tbeg + static_cast<long long>(st) * kKT;
    const int valid = rg.tend - t0 < kKT ? static_cast<int>(rg.tend - t0) : kKT;
    const int buf = st % kDxBufs;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      slab_piece<kSwz16>(src0 + t0 * Wd, Wd, wave * 2 + u, valid, &s_ring[buf][0][0][0], lane);
      slab_piece<kSwz16>(src1 + t0 * Wd, Wd, wave * 2 + u, valid, &s_ring[buf][1][0][0], lane);
      if constexpr (RES) slab_piece<kSwz16>(src2 + t0 * Wd, Wd, wave * 2 + u, valid, &s_ring[buf][kQ - 1][0][0], lane);
    }
  };
  // B operand of k-step ks, token tile tt: slab ks / 8, row tt*16 + lane%16,
  // columns (ks%8)*32 + (lane/16)*8 .. +7
  uint32_t xoff[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) xoff[k] = row_off16(lane & 15, k * 4 + (lane >> 4));
  uint16_t* obase = p.dx_out + kb * kBS + ib + (lane >> 4) * 4;

#pragma unroll
  for (int d = 0; d < kDxBufs - 1; ++d) {
    if (d < rg.n_steps) issue(d);
  }
  for (int st = 0; st < rg.n_steps; ++st) {
    const int ahead = rg.n_steps - 1 - st;
    wait_ring<kDxStores, kDma, kDxBufs - 1, kDxBufs - 2>(st < kDxBufs - 1 ? st : kDxBufs - 1,
                                                         ahead < kDxBufs - 2 ? ahead : kDxBufs - 2);
    // every wave's loads of this step are in LDS, and every wave is done
    // reading the buffer the next issue overwrites (read in step st - 1)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (ahead >= kDxBufs - 1) issue(st + kDxBufs - 1);
    const uint32_t sb = ring0 + static_cast<uint32_t>(st % kDxBufs) * (kQ * kSlabBytes);
    f32x4 acc[2][2];
    if constexpr (RES) {
      // dx_in at row tt*16 + lane%16, channels ib + mt*16 + (lane/16)*4 .. +3
      u32x2 r[2][2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const int row = tt * 16 + (lane & 15);
          const int g = (ib + mt * 16) / 8 + (lane >> 5);
          r[mt][tt] = lds_read8(sb + 2 * kSlabBytes + row_off16(row, g) + ((lane >> 4) & 1) * 8);
        }
      }
      lds_wait<0>(r[0][0], r[0][1]);
      lds_wait<0>(r[1][0], r[1][1]);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          acc[mt][tt] = f32x4{__uint_as_float(r[mt][tt][0] << 16), __uint_as_float(r[mt][tt][0] & 0xFFFF0000u),
                              __uint_as_float(r[mt][tt][1] << 16), __uint_as_float(r[mt][tt][1] & 0xFFFF0000u)};
        }
      }
    } else {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        acc[mt][0] = f32x4{0.f, 0.f, 0.f, 0.f};
        acc[mt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
    // gate-gradient operands of both tiles, at most 8 reads in flight
    u32x4 xb[16][2];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      xb[ks][0] = lds_read16(sb + xoff[ks & 7] + (ks >> 3) * kSlabBytes);
      xb[ks][1] = lds_read16(sb + xoff[ks & 7] + (ks >> 3) * kSlabBytes + 16 * kBS * 2);
    }
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      // in flight: k-steps ks .. min(ks + 3, 15), two reads each
      if (ks <= 12) {
        lds_wait<6>(xb[ks][0], xb[ks][1]);
      } else if (ks == 13) {
        lds_wait<4>(xb[ks][0], xb[ks][1]);
      } else if (ks == 14) {
        lds_wait<2>(xb[ks][0], xb[ks][1]);
      } else {
        lds_wait<0>(xb[ks][0], xb[ks][1]);
      }
      if (ks + 4 < 16) {
        xb[ks + 4][0] = lds_read16(sb + xoff[(ks + 4) & 7] + ((ks + 4) >> 3) * kSlabBytes);
        xb[ks + 4][1] = lds_read16(sb + xoff[(ks + 4) & 7] + ((ks + 4) >> 3) * kSlabBytes + 16 * kBS * 2);
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) acc[mt][tt] = mfma(wr[mt][ks], as_bf16x8(xb[ks][tt]), acc[mt][tt]);
      }
    }
    asm volatile("" ::: "memory");
    const long long t0 = rg.tbeg + static_cast<long long>(st) * kKT;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const long long t = t0 + tt * 16 + (lane & 15);
      if (ahead > 0 || t < rg.tend) {
        uint16_t* orow = obase + t * p.Wd;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          u32x2 v;
          v[0] = pack2(acc[mt][tt][0], acc[mt][tt][1]);
          v[1] = pack2(acc[mt][tt][2], acc[mt][tt][3]);
          *reinterpret_cast<u32x2*>(orow + mt * 16) = v;
        }
      }
    }
    // the stores are issued before the next step's wait counts them
    asm volatile("" ::: "memory");
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

constexpr int kDwBufs = 4;            // LDS ring depth (32 KiB per step)
constexpr int kDwIns = 4;             // 1 KiB loads per wave per step (32 KiB / 8 waves)

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

__global__ __launch_bounds__(kWaves8 * 64) void proj_dw_kernel(ProjDwArgs p) {
  __shared__ __attribute__((aligned(16))) uint16_t s_slab[kDwBufs][2][kKT][kBS];   // [buf][x, dgate][token][col]
  __shared__ float s_cs[4][kBS];
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
  uint32_t roff[kDwIns];                // byte offset of this lane's row from the step's first token
  uint32_t goff[kDwIns];                // byte offset of this lane's granule within the row
  int row[kDwIns];
#pragma unroll
  for (int u = 0; u < kDwIns; ++u) {
    const int ins = wave * kDwIns + u;
    const int r = (ins & 15) * 2 + (lane >> 5);
    const int pos = lane & 31;           // 16-byte granule position in the LDS row
    roff[u] = static_cast<uint32_t>(r) * static_cast<uint32_t>(p.Wd) * 2u;
    goff[u] = static_cast<uint32_t>(((((pos >> 1) ^ (r & 15)) << 1) | (pos & 1)) * 16);
    row[u] = r;
  }
  // loads of step `st`; rows past the range's end read zeros
  auto issue = [=](int st) {
    const long long t0 = tbeg + static_cast<long long>(st) * kKT;
    const int valid = tend - t0 < kKT ? static_cast<int>(tend - t0) : kKT;
#pragma unroll
    for (int u = 0; u < kDwIns; ++u) {
      const int ins = wave * kDwIns + u;
      const char* sb = reinterpret_cast<const char*>(((ins >> 4) == 0 ? base_x : base_g) + t0 * p.Wd);
      const char* rp = row[u] < valid ? sb + roff[u] : reinterpret_cast<const char*>(g_zero_row);
      lds_dma16(rp + goff[u], &s_slab[st % kDwBufs][ins >> 4][(ins & 15) * 2][0]);
    }
  };

  // LDS byte addresses of this lane's operand reads in ring buffer 0
  const uint32_t ring0 = lds_addr(&s_slab[0][0][0][0]);
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

// token ranges for a kernel with `wgs` workgroups per range: about one
// workgroup per CU (each holds a whole CU's worth of registers), no empty range
int range_count(long long T, int wgs) {
  const long long steps = (T + kKT - 1) / kKT;
  long long s = 256 / wgs;
  if (s < 1) s = 1;
  if (s > steps) s = steps;
  const long long per = (steps + s - 1) / s;
  return static_cast<int>((steps + per - 1) / per);
}

long long range_per(long long T, int ranges) {
  const long long steps = (T + kKT - 1) / kKT;
  return ((steps + ranges - 1) / ranges) * kKT;
}

int dw_splits(long long T, int nb) { return range_count(T, 2 * nb); }

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
  a.nb = nb;
  a.ranges = range_count(tokens, nb);
  a.per = range_per(tokens, a.ranges);
  hipLaunchKernelGGL(proj_fwd_kernel, dim3(static_cast<unsigned>(a.ranges) * nb), dim3(kWaves8 * 64), 0,
                     static_cast<hipStream_t>(stream), a);
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
  w.per = range_per(tokens, sw);
  w.part_w = static_cast<float*>(workspace);
  w.part_b = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                      round_up(static_cast<size_t>(sw) * nb * 2 * kBS * kBS * sizeof(float), 256));
  w.T = tokens;
  w.Wd = static_cast<int>(width);
  w.nb = nb;
  w.splits = sw;
  const long long pairs = static_cast<long long>(sw) * nb;
  hipLaunchKernelGGL(proj_dw_kernel, dim3(static_cast<unsigned>(((pairs + 7) / 8) * 16)), dim3(kWaves8 * 64), 0,
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
  d.nb = nb;
  d.ranges = range_count(tokens, nb);
  d.per = range_per(tokens, d.ranges);
  if (dx_in != nullptr) {
    hipLaunchKernelGGL(proj_dx_kernel<true>, dim3(static_cast<unsigned>(d.ranges) * nb), dim3(kWaves8 * 64), 0, st,
                       d);
  } else {
    hipLaunchKernelGGL(proj_dx_kernel<false>, dim3(static_cast<unsigned>(d.ranges) * nb), dim3(kWaves8 * 64), 0, st,
                       d);
  }
  return launch_status();
}

}  // extern "C"
