// RG-LRU scan, forward and backward, for gfx950 (CDNA4).
//
// Method: the fused operator of the Fattori comparison page (sigmoid input and
// recurrence gates, softplus(a_param) dynamic decay, stationary square-root
// multiplier, input-gated write, state-stationary recurrence, custom backward
// with the reverse recurrence and pointwise derivatives), with the canonical
// reset tokens and initial state its "Semantic limits" list calls for, and an
// exact time-parallel chunked form with partial chunks (the page's closing
// paragraph). The equations are stated in include/rglru.h.
//
// Design (one launch per direction):
//  * A workgroup owns a tile: one batch row b, a strip of 64*V channels (V
//    consecutive channels per lane, so every wave load is a contiguous run of
//    64*V channels) and a time chunk of NW*TS steps (TS steps per wave).
//  * Phase 1: each lane streams its TS steps of x, gate_x, gate_a straight
//    into registers, evaluates the gates once, keeps (alpha, write) per step
//    and reduces them to the affine map h_in -> R ? B : A*h_in + B of its
//    steps (R: a reset token inside, so h_in no longer matters).
//  * The waves' maps are composed through LDS into the tile's map. Wave 0
//    publishes it and runs a decoupled look-back over the tiles of earlier
//    chunks of the same (b, strip) to obtain the carry entering the tile,
//    then publishes the carry leaving the tile.
//  * Phase 3: every wave applies its carry and replays its steps from
//    registers, storing h (and the float32 checkpoint every 8 steps).
//  The inputs are read once and the outputs written once. The backward is the
//  mirror image in reverse time; it recomputes the gates from the inputs and
//  the checkpointed carry instead of reading saved gates or states.
//
// Look-back slots. Every published value is a 64-bit word: high half = tag of
// the current call, low half = a float32. Words are written and polled with
// relaxed atomics at agent scope, which the gfx950 memory model makes coherent
// across the XCDs' L2s without fences (no L2 write-back of unrelated data).
// The tag is 1 + the call counter kept in the workspace header; the workgroup
// that finishes last advances it, so stale words of earlier calls can never
// look ready and the workspace never needs clearing between calls. Tiles are
// handed out by an atomic ticket in chunk order, so every tile a workgroup
// waits on belongs to a workgroup that is already running.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>
#include <math.h>

#include <initializer_list>
#include <type_traits>

#include "common.h"

namespace rglru {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kCkpt = RGLRU_CKPT_STEPS;
constexpr unsigned kSpinLimit = 1u << 20;
constexpr size_t kHeaderBytes = 256;
constexpr int kMaxStrip = 512;   // widest channel strip of any variant (64 lanes * 8)

// Widest vector (channels per lane) the forward and backward may use; the
// host picks the widest one that divides W and matches the pointers' alignment.
#ifndef RGLRU_FWD_VMAX
#define RGLRU_FWD_VMAX 4
#endif
#ifndef RGLRU_BWD_VMAX
#define RGLRU_BWD_VMAX 2
#endif

// ------------------------------------------------------------------ io access

struct F32 {
  using elem = float;
};
struct BF16 {
  using elem = uint16_t;
};

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int BYTES> struct Raw;
template <> struct Raw<2> { using T = uint16_t; };
template <> struct Raw<4> { using T = uint32_t; };
template <> struct Raw<8> { using T = u32x2; };
template <> struct Raw<16> { using T = u32x4; };

// V consecutive io elements of one row, moved as a single vector access.
template <typename IO, int V>
struct Io {
  using elem = typename IO::elem;
  static constexpr int kBytes = V * static_cast<int>(sizeof(elem));
  using R = typename Raw<kBytes>::T;
  union U {
    R r;
    elem e[V];
  };

  static __device__ __forceinline__ R load(const void* base, long long off) {
    return *reinterpret_cast<const R*>(reinterpret_cast<const elem*>(base) + off);
  }
  static __device__ __forceinline__ void store(void* base, long long off, R r) {
    *reinterpret_cast<R*>(reinterpret_cast<elem*>(base) + off) = r;
  }
  static __device__ __forceinline__ void unpack(R r, float (&v)[V]) {
    U u;
    u.r = r;
#pragma unroll
    for (int j = 0; j < V; ++j) {
      if constexpr (std::is_same<IO, F32>::value) {
        v[j] = u.e[j];
      } else {
        v[j] = bf16_bits_to_f32(u.e[j]);
      }
    }
  }
  static __device__ __forceinline__ R pack(const float (&v)[V]) {
    U u;
    if constexpr (std::is_same<IO, F32>::value) {
#pragma unroll
      for (int j = 0; j < V; ++j) u.e[j] = v[j];
    } else if constexpr (V == 1) {
      u.e[0] = f32_to_bf16(v[0]);
    } else {
#pragma unroll
      for (int j = 0; j < V; j += 2) {
        uint32_t w = f32x2_to_bf16x2(v[j], v[j + 1]);
        u.e[j] = static_cast<uint16_t>(w & 0xFFFFu);
        u.e[j + 1] = static_cast<uint16_t>(w >> 16);
      }
    }
    return u.r;
  }
};

template <int V>
__device__ __forceinline__ void load_f32v(const float* p, float (&v)[V]) {
  if constexpr (V == 4) {
    float4 t = *reinterpret_cast<const float4*>(p);
    v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
  } else if constexpr (V == 2) {
    float2 t = *reinterpret_cast<const float2*>(p);
    v[0] = t.x; v[1] = t.y;
  } else {
#pragma unroll
    for (int j = 0; j < V; ++j) v[j] = p[j];
  }
}

template <int V>
__device__ __forceinline__ void store_f32v(float* p, const float (&v)[V]) {
  if constexpr (V == 4) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  } else if constexpr (V == 2) {
    *reinterpret_cast<float2*>(p) = make_float2(v[0], v[1]);
  } else {
#pragma unroll
    for (int j = 0; j < V; ++j) p[j] = v[j];
  }
}

// ------------------------------------------------------------------ pointwise math

// Logistic function: 1 / (1 + 2^(-z log2 e)). Saturates to exactly 0 and 1.
__device__ __forceinline__ float sigmoid_f(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-kLog2e * z));
}

// 1 - e^l for l <= 0, given a = e^l. Near 0 it is the Taylor series of
// -expm1(l) through l^8 (relative truncation error below 1e-9 for
// |l| < ln2/2), so the stationary factor sqrt(1 - a^2) keeps full float32
// precision when a is close to 1; elsewhere 1 - a loses at most one bit.
__device__ __forceinline__ float one_minus_exp(float l, float a) {
  float q = 1.0f / 40320.0f;
  q = fmaf(q, l, 1.0f / 5040.0f);
  q = fmaf(q, l, 1.0f / 720.0f);
  q = fmaf(q, l, 1.0f / 120.0f);
  q = fmaf(q, l, 1.0f / 24.0f);
  q = fmaf(q, l, 1.0f / 6.0f);
  q = fmaf(q, l, 0.5f);
  q = fmaf(q, l, 1.0f);
  const float near0 = -l * q;
  return (l > -0.34657359f) ? near0 : 1.0f - a;
}

// Per-channel decay constants: cs = -c * softplus(lambda), k2 = cs * log2 e.
__device__ __forceinline__ void channel_consts(float lam, float c, float& cs, float& k2) {
  const float s = fmaxf(lam, 0.0f) + log1pf(expf(-fabsf(lam)));
  cs = -c * s;
  k2 = cs * kLog2e;
}

// ------------------------------------------------------------------ look-back slots

__device__ __forceinline__ void publish(u64* slot, size_t idx, unsigned tag, uint32_t bits) {
  const u64 w = (static_cast<u64>(tag) << 32) | static_cast<u64>(bits);
  __hip_atomic_store(slot + idx, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ u64 poll(const u64* slot, size_t idx) {
  return __hip_atomic_load(slot + idx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ bool tagged(u64 w, unsigned tag) {
  return static_cast<unsigned>(w >> 32) == tag;
}

// The A of a published map carries the reset flag in its sign bit (A >= 0
// otherwise; a NaN A is stored as the positive quiet NaN).
__device__ __forceinline__ uint32_t encode_a(float A, bool R) {
  if (R) return 0x80000000u;
  return (A != A) ? 0x7FC00000u : __float_as_uint(A);
}

struct Header {
  u64 counter;     // (call counter << 32) | tickets handed out in the running call
  unsigned done;   // workgroups finished in the running call
  unsigned err;    // sticky error bits
};

// LDS of the windowed look-back: one predecessor per wave and round.
template <int V, int NW>
struct LookSmem {
  float a[NW][64 * V];
  float b[NW][64 * V];
  float h[NW][64 * V];
  unsigned char st[NW][64];   // bit 0: map ready, bit 1: carry ready, bit 2: map has a reset
  int done[64];
  int pending;
};

// Carry entering a tile (valid in wave 0 on return). Called by every thread
// of the workgroup. In each round wave w polls the predecessor at distance
// w + 1 (tiles of earlier chunks of the same row in the forward, of later
// chunks in the backward), so one memory round trip covers NW predecessors.
// Wave 0 then looks for the nearest predecessor whose outgoing carry is
// known (published, or fixed by a reset inside it) with every map between
// published, and applies those maps oldest first with the very fma the
// predecessors use for their own outgoing carries. The carry is therefore
// bit-identical to the serial chain whatever the timing: results are
// deterministic run to run.
// `self` is the slot index of this lane's first channel in this tile,
// `stride` the slot distance between consecutive predecessors, `npred` how
// many exist, `init` the carry before the first chunk.
template <int V, int NW>
__device__ __forceinline__ void look_back(LookSmem<V, NW>& sm, const u64* slot_a, const u64* slot_b,
                                          const u64* slot_h, long long self, long long stride, int npred,
                                          unsigned tag, bool active, int wave, int lane,
                                          const float (&init)[V], float (&carry)[V], unsigned* err) {
  bool done = !active;
#pragma unroll
  for (int j = 0; j < V; ++j) carry[j] = 0.0f;
  if (wave == 0) sm.done[lane] = done ? 1 : 0;
  __syncthreads();
  for (unsigned round = 0;; ++round) {
    unsigned char st = 0;
    if (sm.done[lane] == 0 && wave < npred) {
      const long long q = self - static_cast<long long>(wave + 1) * stride;
      u64 wh[V];
      bool ok = true;
#pragma unroll
      for (int j = 0; j < V; ++j) {
        wh[j] = poll(slot_h, q + j);
        ok = ok && tagged(wh[j], tag);
      }
      if (ok) {
        st = 2;
#pragma unroll
        for (int j = 0; j < V; ++j) sm.h[wave][lane * V + j] = __uint_as_float(static_cast<uint32_t>(wh[j]));
      } else {
        u64 wa[V], wb[V];
        ok = true;
#pragma unroll
        for (int j = 0; j < V; ++j) {
          wa[j] = poll(slot_a, q + j);
          wb[j] = poll(slot_b, q + j);
          ok = ok && tagged(wa[j], tag) && tagged(wb[j], tag);
        }
        if (ok) {
          st = ((static_cast<uint32_t>(wa[0]) >> 31) != 0) ? 5 : 1;
#pragma unroll
          for (int j = 0; j < V; ++j) {
            sm.a[wave][lane * V + j] = __uint_as_float(static_cast<uint32_t>(wa[j]) & 0x7FFFFFFFu);
            sm.b[wave][lane * V + j] = __uint_as_float(static_cast<uint32_t>(wb[j]));
          }
        }
      }
    }
    sm.st[wave][lane] = st;
    __syncthreads();
    if (wave == 0) {
      if (!done) {
        // nearest resolvable start: a published carry, a reset map, or the sequence start
        int start = -1;
        int kind = 0;   // 1: published carry, 2: reset map, 3: initial carry
        for (int w = 0; w < NW; ++w) {
          if (w >= npred) {
            start = w;
            kind = 3;
            break;
          }
          const unsigned char sw = sm.st[w][lane];
          if (sw & 2) {
            start = w;
            kind = 1;
            break;
          }
          if ((sw & 1) == 0) break;
          if (sw & 4) {
            start = w;
            kind = 2;
            break;
          }
        }
        if (start >= 0) {
          float hv[V];
#pragma unroll
          for (int j = 0; j < V; ++j) {
            hv[j] = kind == 1 ? sm.h[start][lane * V + j] : (kind == 2 ? sm.b[start][lane * V + j] : init[j]);
          }
          for (int w = start - 1; w >= 0; --w) {
#pragma unroll
            for (int j = 0; j < V; ++j) hv[j] = fmaf(sm.a[w][lane * V + j], hv[j], sm.b[w][lane * V + j]);
          }
#pragma unroll
          for (int j = 0; j < V; ++j) carry[j] = hv[j];
          done = true;
        } else if (round >= kSpinLimit) {
          atomicOr(err, 1u);
          done = true;
        }
        sm.done[lane] = done ? 1 : 0;
      }
      const bool any = __ballot(!done) != 0ull;
      if (lane == 0) sm.pending = any ? 1 : 0;
    }
    __syncthreads();
    if (sm.pending == 0) break;
    __builtin_amdgcn_s_sleep(1);
  }
}

// Called once per workgroup at its end: the last one re-arms the ticket
// counter and advances the call counter (and with it the slot tag).
__device__ __forceinline__ void finish_call(Header* hdr, unsigned n_tiles) {
  const unsigned prev = atomicAdd(&hdr->done, 1u);
  if (prev == n_tiles - 1) {
    atomicExch(&hdr->done, 0u);
    atomicAdd(&hdr->counter, (1ull << 32) - static_cast<u64>(n_tiles));
  }
}

// Ticket of this workgroup: (tile index, slot tag), wave-uniform.
__device__ __forceinline__ void take_ticket(Header* hdr, unsigned* s_ticket, unsigned& tile, unsigned& tag) {
  if (threadIdx.x == 0) {
    const u64 v = atomicAdd(&hdr->counter, 1ull);
    s_ticket[0] = static_cast<unsigned>(v);
    s_ticket[1] = static_cast<unsigned>(v >> 32) + 1u;
  }
  __syncthreads();
  tile = __builtin_amdgcn_readfirstlane(s_ticket[0]);
  tag = __builtin_amdgcn_readfirstlane(s_ticket[1]);
}

// ------------------------------------------------------------------ forward

struct FwdArgs {
  const void* x;
  const void* gx;
  const void* ga;
  const float* lam;
  const uint8_t* reset;
  const float* h0;
  void* h;
  float* h_last;
  float* ckpt;
  Header* hdr;
  u64* slot_a;
  u64* slot_b;
  u64* slot_h;
  long long L;
  long long n_ckpt;
  int B;
  int W;
  int n_strips;
  int n_chunks;
  unsigned n_tiles;
  float c;
};

template <typename IO, int V, int TS, int NW, int WPE>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(WPE)))
void fwd_kernel(FwdArgs p) {
  static_assert(TS % kCkpt == 0, "a wave's steps must cover whole checkpoint intervals");
  constexpr int SW = 64 * V;
  constexpr int T = TS * NW;
  using io = Io<IO, V>;
  using R_t = typename io::R;

  __shared__ unsigned s_ticket[2];
  __shared__ float s_A[NW][SW];
  __shared__ float s_B[NW][SW];
  __shared__ unsigned s_R[NW];
  __shared__ float s_carry[SW];
  __shared__ LookSmem<V, NW> s_look;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  unsigned tile, tag;
  take_ticket(p.hdr, s_ticket, tile, tag);
  const unsigned rows = static_cast<unsigned>(p.B) * static_cast<unsigned>(p.n_strips);
  const int chunk = static_cast<int>(tile / rows);
  const int row = static_cast<int>(tile - static_cast<unsigned>(chunk) * rows);
  const int b = row / p.n_strips;
  const int strip = row - b * p.n_strips;
  const int ch = strip * SW + lane * V;
  const bool active = ch < p.W;
  const long long t0 = static_cast<long long>(chunk) * T + static_cast<long long>(wave) * TS;
  const long long rem = p.L - t0;
  const int nvalid = rem <= 0 ? 0 : (rem >= TS ? TS : static_cast<int>(rem));
  const long long rowbase = static_cast<long long>(b) * p.L;
  const long long W = p.W;

  // reset flags of this wave's steps as a wave-uniform bit mask
  unsigned rmask = 0;
  if (p.reset != nullptr) {
    const bool f = lane < nvalid && p.reset[rowbase + t0 + lane] != 0;
    rmask = static_cast<unsigned>(__ballot(f));
  }

  // phase 1: stream the steps in
  R_t rx[TS], rgx[TS], rga[TS];
#pragma unroll
  for (int k = 0; k < TS; ++k) {
    if (active && k < nvalid) {
      const long long off = (rowbase + t0 + k) * W + ch;
      rx[k] = io::load(p.x, off);
      rgx[k] = io::load(p.gx, off);
      rga[k] = io::load(p.ga, off);
    } else {
      rx[k] = R_t{};
      rgx[k] = R_t{};
      rga[k] = R_t{};
    }
  }
  float cs[V], k2[V];
#pragma unroll
  for (int j = 0; j < V; ++j) {
    cs[j] = 0.0f;
    k2[j] = 0.0f;
    if (active) channel_consts(p.lam[ch + j], p.c, cs[j], k2[j]);
  }

  float al[TS][V], u[TS][V];
#pragma unroll
  for (int k = 0; k < TS; ++k) {
    float xv[V], gxv[V], gav[V];
    io::unpack(rx[k], xv);
    io::unpack(rgx[k], gxv);
    io::unpack(rga[k], gav);
    const bool rs = (rmask >> k) & 1u;
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const float i = sigmoid_f(gxv[j]);
      const float r = sigmoid_f(gav[j]);
      const float l = cs[j] * r;
      const float a = __builtin_amdgcn_exp2f(k2[j] * r);
      const float m = __builtin_amdgcn_sqrtf(one_minus_exp(l, a) * (1.0f + a));
      al[k][j] = rs ? 0.0f : a;
      u[k][j] = (rs ? 1.0f : m) * i * xv[j];
    }
  }

  // this wave's map
  float A[V], Bv[V];
#pragma unroll
  for (int j = 0; j < V; ++j) {
    A[j] = 1.0f;
    Bv[j] = 0.0f;
  }
#pragma unroll
  for (int k = 0; k < TS; ++k) {
    if (k < nvalid) {
      const bool rs = (rmask >> k) & 1u;
#pragma unroll
      for (int j = 0; j < V; ++j) {
        Bv[j] = rs ? u[k][j] : fmaf(al[k][j], Bv[j], u[k][j]);
        A[j] *= al[k][j];
      }
    }
  }
#pragma unroll
  for (int j = 0; j < V; ++j) {
    s_A[wave][lane * V + j] = A[j];
    s_B[wave][lane * V + j] = Bv[j];
  }
  if (lane == 0) s_R[wave] = rmask != 0u ? 1u : 0u;
  __syncthreads();

  // the tile's map (every wave computes it; wave 0 publishes it)
  float GA[V], GB[V];
  bool GR = false;
#pragma unroll
  for (int j = 0; j < V; ++j) {
    GA[j] = 1.0f;
    GB[j] = 0.0f;
  }
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const bool Rw = s_R[w] != 0u;
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const float Aw = s_A[w][lane * V + j];
      const float Bw = s_B[w][lane * V + j];
      GB[j] = Rw ? Bw : fmaf(Aw, GB[j], Bw);
      GA[j] *= Aw;
    }
    GR = GR || Rw;
  }
  const size_t sbase = static_cast<size_t>(tile) * SW + static_cast<size_t>(lane) * V;
  const bool has_succ = chunk < p.n_chunks - 1;
  float init[V], carry[V];
#pragma unroll
  for (int j = 0; j < V; ++j) init[j] = (active && p.h0 != nullptr) ? p.h0[b * W + ch + j] : 0.0f;
  if (chunk == 0) {
#pragma unroll
    for (int j = 0; j < V; ++j) carry[j] = init[j];
  } else {
    if (wave == 0 && active && has_succ) {
#pragma unroll
      for (int j = 0; j < V; ++j) {
        publish(p.slot_a, sbase + j, tag, encode_a(GA[j], GR));
        publish(p.slot_b, sbase + j, tag, __float_as_uint(GB[j]));
      }
    }
    look_back<V, NW>(s_look, p.slot_a, p.slot_b, p.slot_h, static_cast<long long>(sbase),
                     static_cast<long long>(rows) * SW, chunk, tag, active, wave, lane, init, carry,
                     &p.hdr->err);
  }
  if (wave == 0 && active) {
    if (has_succ) {
#pragma unroll
      for (int j = 0; j < V; ++j) {
        const float hout = GR ? GB[j] : fmaf(GA[j], carry[j], GB[j]);
        publish(p.slot_h, sbase + j, tag, __float_as_uint(hout));
      }
    }
#pragma unroll
    for (int j = 0; j < V; ++j) s_carry[lane * V + j] = carry[j];
  }
  __syncthreads();

  // phase 3: replay from the carry entering this wave
  if (active) {
    float hc[V];
#pragma unroll
    for (int j = 0; j < V; ++j) hc[j] = s_carry[lane * V + j];
    for (int w = 0; w < wave; ++w) {
      const bool Rw = s_R[w] != 0u;
#pragma unroll
      for (int j = 0; j < V; ++j) {
        hc[j] = Rw ? s_B[w][lane * V + j] : fmaf(s_A[w][lane * V + j], hc[j], s_B[w][lane * V + j]);
      }
    }
#pragma unroll
    for (int k = 0; k < TS; ++k) {
      if (k < nvalid) {
        const long long t = t0 + k;
        if (p.ckpt != nullptr && (k % kCkpt) == 0) {
          store_f32v<V>(p.ckpt + (static_cast<long long>(b) * p.n_ckpt + t / kCkpt) * W + ch, hc);
        }
        const bool rs = (rmask >> k) & 1u;
#pragma unroll
        for (int j = 0; j < V; ++j) hc[j] = rs ? u[k][j] : fmaf(al[k][j], hc[j], u[k][j]);
        io::store(p.h, (rowbase + t) * W + ch, io::pack(hc));
      }
    }
    if (p.h_last != nullptr && nvalid > 0 && t0 + nvalid == p.L) {
      store_f32v<V>(p.h_last + b * W + ch, hc);
    }
  }
  if (threadIdx.x == 0) finish_call(p.hdr, p.n_tiles);
}

// ------------------------------------------------------------------ backward

struct BwdArgs {
  const void* x;
  const void* gx;
  const void* ga;
  const float* lam;
  const uint8_t* reset;
  const float* ckpt;
  const void* dh;
  const float* dh_last;
  void* dx;
  void* dgx;
  void* dga;
  float* dlam;
  float* dh0;
  Header* hdr;
  u64* slot_a;
  u64* slot_b;
  u64* slot_h;
  u64* slot_p;       // per-tile lambda-gradient partials
  long long L;
  long long n_ckpt;
  int B;
  int W;
  int n_strips;
  int n_chunks;
  unsigned n_tiles;
  float c;
};

// Every wave covers exactly one checkpoint interval, whose entering carry the
// forward stored. Tiles are handed out from the last chunk backwards.
template <typename IO, int V, int NW, int WPE>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(WPE)))
void bwd_kernel(BwdArgs p) {
  constexpr int TS = kCkpt;
  constexpr int SW = 64 * V;
  constexpr int T = TS * NW;
  using io = Io<IO, V>;
  using R_t = typename io::R;

  __shared__ unsigned s_ticket[2];
  __shared__ float s_A[NW][SW];
  __shared__ float s_B[NW][SW];
  __shared__ unsigned s_R[NW];
  __shared__ float s_carry[SW];
  __shared__ LookSmem<V, NW> s_look;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  unsigned tile, tag;
  take_ticket(p.hdr, s_ticket, tile, tag);
  const unsigned rows = static_cast<unsigned>(p.B) * static_cast<unsigned>(p.n_strips);
  const int crev = static_cast<int>(tile / rows);          // 0 = last chunk in time
  const int row = static_cast<int>(tile - static_cast<unsigned>(crev) * rows);
  const int chunk = p.n_chunks - 1 - crev;
  const int b = row / p.n_strips;
  const int strip = row - b * p.n_strips;
  const int ch = strip * SW + lane * V;
  const bool active = ch < p.W;
  const long long t0 = static_cast<long long>(chunk) * T + static_cast<long long>(wave) * TS;
  const long long rem = p.L - t0;
  const int nvalid = rem <= 0 ? 0 : (rem >= TS ? TS : static_cast<int>(rem));
  const long long rowbase = static_cast<long long>(b) * p.L;
  const long long W = p.W;

  unsigned rmask = 0;
  if (p.reset != nullptr) {
    const bool f = lane < nvalid && p.reset[rowbase + t0 + lane] != 0;
    rmask = static_cast<unsigned>(__ballot(f));
  }

  R_t rx[TS], rgx[TS], rga[TS], rdh[TS];
#pragma unroll
  for (int k = 0; k < TS; ++k) {
    if (active && k < nvalid) {
      const long long off = (rowbase + t0 + k) * W + ch;
      rx[k] = io::load(p.x, off);
      rgx[k] = io::load(p.gx, off);
      rga[k] = io::load(p.ga, off);
      rdh[k] = io::load(p.dh, off);
    } else {
      rx[k] = R_t{};
      rgx[k] = R_t{};
      rga[k] = R_t{};
      rdh[k] = R_t{};
    }
  }
  float h[V];
#pragma unroll
  for (int j = 0; j < V; ++j) h[j] = 0.0f;
  if (active && nvalid > 0) load_f32v<V>(p.ckpt + (static_cast<long long>(b) * p.n_ckpt + t0 / kCkpt) * W + ch, h);
  float cs[V], k2[V];
#pragma unroll
  for (int j = 0; j < V; ++j) {
    cs[j] = 0.0f;
    k2[j] = 0.0f;
    if (active) channel_consts(p.lam[ch + j], p.c, cs[j], k2[j]);
  }

  // Recompute the forward through this wave's steps and turn every step into
  // the coefficients the reverse pass needs:
  //   g = G + dh;  dx = g*cx;  dgate_x = g*cgx;  dgate_a = g*cga;
  //   lambda-gradient partial += g*cl;  G <- alpha*g  (0 after a reset token)
  // with dl = g * a*(h_prev - a*i*x/m) off reset tokens (0 on them).
  float cx[TS][V], cgx[TS][V], cga[TS][V], cl[TS][V], al[TS][V], dhv[TS][V];
#pragma unroll
  for (int k = 0; k < TS; ++k) {
    float xv[V], gxv[V], gav[V];
    io::unpack(rx[k], xv);
    io::unpack(rgx[k], gxv);
    io::unpack(rga[k], gav);
    io::unpack(rdh[k], dhv[k]);
    const bool rs = (rmask >> k) & 1u;
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const float i = sigmoid_f(gxv[j]);
      const float r = sigmoid_f(gav[j]);
      const float l = cs[j] * r;
      const float a = __builtin_amdgcn_exp2f(k2[j] * r);
      const float w = one_minus_exp(l, a) * (1.0f + a);   // 1 - a^2
      const float rsq = __builtin_amdgcn_rsqf(w);          // 1 / m
      const float m = w * rsq;
      const float mult = rs ? 1.0f : m;
      const float ix = i * xv[j];
      const float z = rs ? 0.0f : a * (h[j] - a * ix * rsq);
      const float uw = mult * ix;
      h[j] = rs ? uw : fmaf(a, h[j], uw);
      cx[k][j] = mult * i;
      cgx[k][j] = mult * ix * (1.0f - i);
      const float rr = r * (1.0f - r);
      cga[k][j] = z * cs[j] * rr;
      cl[k][j] = z * r;
      al[k][j] = rs ? 0.0f : a;
    }
  }

  // this wave's reverse map G_in -> G_out (G_out = carry handed to the step before the wave)
  float A[V], Bv[V];
#pragma unroll
  for (int j = 0; j < V; ++j) {
    A[j] = 1.0f;
    Bv[j] = 0.0f;
  }
#pragma unroll
  for (int k = TS - 1; k >= 0; --k) {
    if (k < nvalid) {
      const bool rs = (rmask >> k) & 1u;
#pragma unroll
      for (int j = 0; j < V; ++j) {
        const float gB = Bv[j] + dhv[k][j];
        Bv[j] = rs ? 0.0f : al[k][j] * gB;
        A[j] = rs ? 0.0f : al[k][j] * A[j];
      }
    }
  }
#pragma unroll
  for (int j = 0; j < V; ++j) {
    s_A[wave][lane * V + j] = A[j];
    s_B[wave][lane * V + j] = Bv[j];
  }
  if (lane == 0) s_R[wave] = rmask != 0u ? 1u : 0u;
  __syncthreads();

  float GA[V], GB[V];
  bool GR = false;
#pragma unroll
  for (int j = 0; j < V; ++j) {
    GA[j] = 1.0f;
    GB[j] = 0.0f;
  }
#pragma unroll
  for (int w = NW - 1; w >= 0; --w) {
    const bool Rw = s_R[w] != 0u;
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const float Aw = s_A[w][lane * V + j];
      const float Bw = s_B[w][lane * V + j];
      GB[j] = Rw ? Bw : fmaf(Aw, GB[j], Bw);
      GA[j] *= Aw;
    }
    GR = GR || Rw;
  }
  const size_t sbase = static_cast<size_t>(tile) * SW + static_cast<size_t>(lane) * V;
  const bool has_succ = crev < p.n_chunks - 1;
  float init[V], carry[V];
#pragma unroll
  for (int j = 0; j < V; ++j) init[j] = (active && p.dh_last != nullptr) ? p.dh_last[b * W + ch + j] : 0.0f;
  if (crev == 0) {
#pragma unroll
    for (int j = 0; j < V; ++j) carry[j] = init[j];
  } else {
    if (wave == 0 && active && has_succ) {
#pragma unroll
      for (int j = 0; j < V; ++j) {
        publish(p.slot_a, sbase + j, tag, encode_a(GA[j], GR));
        publish(p.slot_b, sbase + j, tag, __float_as_uint(GB[j]));
      }
    }
    look_back<V, NW>(s_look, p.slot_a, p.slot_b, p.slot_h, static_cast<long long>(sbase),
                     static_cast<long long>(rows) * SW, crev, tag, active, wave, lane, init, carry,
                     &p.hdr->err);
  }
  if (wave == 0 && active) {
    if (has_succ) {
#pragma unroll
      for (int j = 0; j < V; ++j) {
        const float gout = GR ? GB[j] : fmaf(GA[j], carry[j], GB[j]);
        publish(p.slot_h, sbase + j, tag, __float_as_uint(gout));
      }
    }
#pragma unroll
    for (int j = 0; j < V; ++j) s_carry[lane * V + j] = carry[j];
  }
  __syncthreads();

  float dl_acc[V];
#pragma unroll
  for (int j = 0; j < V; ++j) dl_acc[j] = 0.0f;
  if (active) {
    float G[V];
#pragma unroll
    for (int j = 0; j < V; ++j) G[j] = s_carry[lane * V + j];
    for (int w = NW - 1; w > wave; --w) {
      const bool Rw = s_R[w] != 0u;
#pragma unroll
      for (int j = 0; j < V; ++j) {
        G[j] = Rw ? s_B[w][lane * V + j] : fmaf(s_A[w][lane * V + j], G[j], s_B[w][lane * V + j]);
      }
    }
#pragma unroll
    for (int k = TS - 1; k >= 0; --k) {
      if (k < nvalid) {
        const bool rs = (rmask >> k) & 1u;
        float ox[V], ogx[V], oga[V];
#pragma unroll
        for (int j = 0; j < V; ++j) {
          const float g = G[j] + dhv[k][j];
          ox[j] = g * cx[k][j];
          ogx[j] = g * cgx[k][j];
          oga[j] = g * cga[k][j];
          dl_acc[j] = fmaf(g, cl[k][j], dl_acc[j]);
          G[j] = rs ? 0.0f : al[k][j] * g;
        }
        const long long off = (rowbase + t0 + k) * W + ch;
        io::store(p.dx, off, io::pack(ox));
        io::store(p.dgx, off, io::pack(ogx));
        io::store(p.dga, off, io::pack(oga));
      }
    }
    if (chunk == 0 && wave == 0 && p.dh0 != nullptr) store_f32v<V>(p.dh0 + b * W + ch, G);
  }

  // the tile's lambda-gradient partial: fixed-order sum over the waves, published tagged
  __syncthreads();
#pragma unroll
  for (int j = 0; j < V; ++j) s_A[wave][lane * V + j] = dl_acc[j];
  __syncthreads();
  if (wave == 0 && active) {
#pragma unroll
    for (int j = 0; j < V; ++j) {
      float s = 0.0f;
      for (int w = 0; w < NW; ++w) s += s_A[w][lane * V + j];
      publish(p.slot_p, sbase + j, tag, __float_as_uint(s));
    }
  }

  // The tile with the largest ticket of its channel strip (chunk 0, last
  // batch row) sums the strip's partials in a fixed order: waves take
  // contiguous runs of (chunk, batch) pairs, then wave 0 adds the runs in
  // wave order. Every partial it waits for belongs to a smaller ticket.
  if (crev == p.n_chunks - 1 && b == p.B - 1) {
    const int n_parts = p.n_chunks * p.B;
    const int per = (n_parts + NW - 1) / NW;
    const int k0 = wave * per;
    const int k1 = k0 + per < n_parts ? k0 + per : n_parts;
    float s[V];
#pragma unroll
    for (int j = 0; j < V; ++j) s[j] = 0.0f;
    bool failed = false;
    if (active) {
      for (int k = k0; k < k1; ++k) {
        const int cr = k / p.B;
        const int bb = k - cr * p.B;
        const long long q = (static_cast<long long>(cr) * rows + static_cast<long long>(bb) * p.n_strips + strip) * SW +
                            static_cast<long long>(lane) * V;
        u64 wv[V];
        unsigned spins = 0;
        while (true) {
          bool ok = true;
#pragma unroll
          for (int j = 0; j < V; ++j) {
            wv[j] = poll(p.slot_p, q + j);
            ok = ok && tagged(wv[j], tag);
          }
          if (ok) break;
          if (++spins > kSpinLimit) {
            failed = true;
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
#pragma unroll
        for (int j = 0; j < V; ++j) s[j] += __uint_as_float(static_cast<uint32_t>(wv[j]));
      }
    }
    if (failed) atomicOr(&p.hdr->err, 1u);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < V; ++j) s_A[wave][lane * V + j] = s[j];
    __syncthreads();
    if (wave == 0 && active) {
#pragma unroll
      for (int j = 0; j < V; ++j) {
        float tot = 0.0f;
        for (int w = 0; w < NW; ++w) tot += s_A[w][lane * V + j];
        const float lm = p.lam[ch + j];
        const float sig = 1.0f / (1.0f + expf(-lm));
        p.dlam[ch + j] = -p.c * sig * tot;
      }
    }
  }
  if (threadIdx.x == 0) finish_call(p.hdr, p.n_tiles);
}

// ------------------------------------------------------------------ host side

struct Geometry {
  int io_bytes;
  int T;          // forward chunk
  int Tb;         // backward chunk
  long long n_ckpt;
  int n_chunks_f;
  int n_chunks_b;
};

bool shape_ok(const rglru_shape_t* s) {
  if (s == nullptr) return false;
  if (s->batch < 1 || s->length < 1 || s->width < 1) return false;
  if (s->io_dtype != RGLRU_IO_F32 && s->io_dtype != RGLRU_IO_BF16) return false;
  if (s->reserved != 0) return false;
  if (!(s->c == s->c) || s->c == INFINITY || s->c == -INFINITY) return false;
  switch (s->chunk) {
    case 0: case 8: case 16: case 32: case 64: case 128: case 256: break;
    default: return false;
  }
  // index arithmetic limits: batch and width fit int, tile counts fit 32 bits
  if (s->batch > (1LL << 24) || s->width > (1LL << 30)) return false;
  const long long strips = ceil_div(s->width, 64);
  const long long tiles = strips * s->batch * ceil_div(s->length, 8);
  if (tiles >= (1LL << 31)) return false;
  return true;
}

Geometry geometry(const rglru_shape_t* s) {
  Geometry g;
  g.io_bytes = s->io_dtype == RGLRU_IO_F32 ? 4 : 2;
  g.T = s->chunk == 0 ? 64 : s->chunk;
  g.Tb = g.T > 128 ? 128 : g.T;
  g.n_ckpt = ceil_div(s->length, kCkpt);
  g.n_chunks_f = static_cast<int>(ceil_div(s->length, g.T));
  g.n_chunks_b = static_cast<int>(ceil_div(s->length, g.Tb));
  return g;
}

// slot words per kind: one per (chunk, b, padded channel)
size_t slot_words(const rglru_shape_t* s, int n_chunks) {
  return static_cast<size_t>(n_chunks) * static_cast<size_t>(s->batch) *
         round_up(static_cast<size_t>(s->width), kMaxStrip);
}

constexpr int kSlotKinds = 4;   // map A, map B, carry, lambda-gradient partial

size_t ws_bytes(const rglru_shape_t* s, int n_chunks) {
  return kHeaderBytes + kSlotKinds * round_up(slot_words(s, n_chunks) * 8, 256);
}

size_t fwd_ws(const rglru_shape_t* s) { return ws_bytes(s, geometry(s).n_chunks_f); }
size_t bwd_ws(const rglru_shape_t* s) { return ws_bytes(s, geometry(s).n_chunks_b); }

struct Slots {
  Header* hdr;
  u64* a;
  u64* b;
  u64* h;
  u64* p;
};

Slots slots_in(void* ws, size_t words) {
  char* base = static_cast<char*>(ws);
  const size_t kind = round_up(words * 8, 256);
  Slots sl;
  sl.hdr = reinterpret_cast<Header*>(base);
  sl.a = reinterpret_cast<u64*>(base + kHeaderBytes);
  sl.b = reinterpret_cast<u64*>(base + kHeaderBytes + kind);
  sl.h = reinterpret_cast<u64*>(base + kHeaderBytes + 2 * kind);
  sl.p = reinterpret_cast<u64*>(base + kHeaderBytes + 3 * kind);
  return sl;
}

// Largest V in {vmax, ..., 1} (powers of two) that divides W and to which
// every io pointer (V elements) and float pointer (V floats) is aligned.
int pick_vec(int vmax, long long W, int io_bytes, std::initializer_list<const void*> io_ptrs,
             std::initializer_list<const void*> f32_ptrs) {
  for (int v = vmax; v > 1; v >>= 1) {
    if (W % v != 0) continue;
    bool ok = true;
    for (const void* q : io_ptrs) ok = ok && (q == nullptr || aligned_to(q, static_cast<size_t>(v) * io_bytes));
    for (const void* q : f32_ptrs) ok = ok && (q == nullptr || aligned_to(q, static_cast<size_t>(v) * 4));
    if (ok) return v;
  }
  return 1;
}

// waves per SIMD the register budget is fitted to: two workgroups per CU
constexpr int wpe_for(int nw) { return nw >= 16 ? 4 : (nw >= 2 ? nw / 2 : 1); }

template <typename IO, int V, int TS, int NW>
rglru_status_t launch_fwd(FwdArgs a, hipStream_t stream) {
  a.n_strips = static_cast<int>(ceil_div(a.W, 64 * V));
  a.n_chunks = static_cast<int>(ceil_div(a.L, TS * NW));
  a.n_tiles = static_cast<unsigned>(a.n_chunks) * static_cast<unsigned>(a.B) * static_cast<unsigned>(a.n_strips);
  hipLaunchKernelGGL((fwd_kernel<IO, V, TS, NW, wpe_for(NW)>), dim3(a.n_tiles), dim3(NW * 64), 0, stream, a);
  return launch_status();
}

template <typename IO, int V>
rglru_status_t dispatch_fwd_chunk(int T, FwdArgs a, hipStream_t stream) {
  switch (T) {
    case 8: return launch_fwd<IO, V, 8, 1>(a, stream);
    case 16: return launch_fwd<IO, V, 8, 2>(a, stream);
    case 32: return launch_fwd<IO, V, 8, 4>(a, stream);
    case 64: return launch_fwd<IO, V, 8, 8>(a, stream);
    case 128: return launch_fwd<IO, V, 8, 16>(a, stream);
    default: break;
  }
  return RGLRU_ERR_UNSUPPORTED;
}

template <typename IO>
rglru_status_t dispatch_fwd(int T, int V, FwdArgs a, hipStream_t stream) {
  if (T == 256) {
    // 16 waves of 16 steps: keep the per-lane state within the register budget
    if (V >= 2) return launch_fwd<IO, 2, 16, 16>(a, stream);
    return launch_fwd<IO, 1, 16, 16>(a, stream);
  }
  switch (V) {
    case 4: return dispatch_fwd_chunk<IO, 4>(T, a, stream);
    case 2: return dispatch_fwd_chunk<IO, 2>(T, a, stream);
    default: return dispatch_fwd_chunk<IO, 1>(T, a, stream);
  }
}

template <typename IO, int V, int NW>
rglru_status_t launch_bwd(BwdArgs a, hipStream_t stream) {
  a.n_strips = static_cast<int>(ceil_div(a.W, 64 * V));
  a.n_chunks = static_cast<int>(ceil_div(a.L, kCkpt * NW));
  a.n_tiles = static_cast<unsigned>(a.n_chunks) * static_cast<unsigned>(a.B) * static_cast<unsigned>(a.n_strips);
  hipLaunchKernelGGL((bwd_kernel<IO, V, NW, wpe_for(NW)>), dim3(a.n_tiles), dim3(NW * 64), 0, stream, a);
  return launch_status();
}

template <typename IO, int V>
rglru_status_t dispatch_bwd_chunk(int Tb, BwdArgs a, hipStream_t stream) {
  switch (Tb) {
    case 8: return launch_bwd<IO, V, 1>(a, stream);
    case 16: return launch_bwd<IO, V, 2>(a, stream);
    case 32: return launch_bwd<IO, V, 4>(a, stream);
    case 64: return launch_bwd<IO, V, 8>(a, stream);
    case 128: return launch_bwd<IO, V, 16>(a, stream);
    default: break;
  }
  return RGLRU_ERR_UNSUPPORTED;
}

template <typename IO>
rglru_status_t dispatch_bwd(int Tb, int V, BwdArgs a, hipStream_t stream) {
  if (V >= 2) return dispatch_bwd_chunk<IO, 2>(Tb, a, stream);
  return dispatch_bwd_chunk<IO, 1>(Tb, a, stream);
}

bool io_aligned(const void* p, int io_bytes) { return p == nullptr || aligned_to(p, io_bytes); }
bool f32_aligned(const void* p) { return p == nullptr || aligned_to(p, 4); }

}  // namespace
}  // namespace rglru

using namespace rglru;

extern "C" {

size_t rglru_ckpt_elems(const rglru_shape_t* s) {
  if (!shape_ok(s)) return 0;
  return static_cast<size_t>(s->batch) * static_cast<size_t>(ceil_div(s->length, kCkpt)) *
         static_cast<size_t>(s->width);
}

size_t rglru_fwd_workspace_bytes(const rglru_shape_t* s) { return shape_ok(s) ? fwd_ws(s) : 0; }

size_t rglru_bwd_workspace_bytes(const rglru_shape_t* s) { return shape_ok(s) ? bwd_ws(s) : 0; }

size_t rglru_workspace_bytes(const rglru_shape_t* s) {
  if (!shape_ok(s)) return 0;
  const size_t f = fwd_ws(s), b = bwd_ws(s);
  return f > b ? f : b;
}

rglru_status_t rglru_fwd(const rglru_shape_t* s, const void* x, const void* gate_x, const void* gate_a,
                         const float* lambda, const uint8_t* reset, const float* h0, void* h,
                         float* h_last, float* ckpt, void* workspace, size_t workspace_bytes,
                         void* stream) {
  if (!shape_ok(s)) return RGLRU_ERR_INVALID_ARGUMENT;
  if (!x || !gate_x || !gate_a || !lambda || !h || !workspace) return RGLRU_ERR_INVALID_ARGUMENT;
  const Geometry g = geometry(s);
  if (!io_aligned(x, g.io_bytes) || !io_aligned(gate_x, g.io_bytes) || !io_aligned(gate_a, g.io_bytes) ||
      !io_aligned(h, g.io_bytes) || !f32_aligned(lambda) || !f32_aligned(h0) || !f32_aligned(h_last) ||
      !f32_aligned(ckpt) || !aligned_to(workspace, 256)) {
    return RGLRU_ERR_MISALIGNED;
  }
  if (workspace_bytes < fwd_ws(s)) return RGLRU_ERR_WORKSPACE_TOO_SMALL;

  const int V = pick_vec(RGLRU_FWD_VMAX, s->width, g.io_bytes, {x, gate_x, gate_a, h}, {h0, h_last, ckpt});
  const Slots sl = slots_in(workspace, slot_words(s, g.n_chunks_f));
  FwdArgs a;
  a.x = x;
  a.gx = gate_x;
  a.ga = gate_a;
  a.lam = lambda;
  a.reset = reset;
  a.h0 = h0;
  a.h = h;
  a.h_last = h_last;
  a.ckpt = ckpt;
  a.hdr = sl.hdr;
  a.slot_a = sl.a;
  a.slot_b = sl.b;
  a.slot_h = sl.h;
  a.L = s->length;
  a.n_ckpt = g.n_ckpt;
  a.B = static_cast<int>(s->batch);
  a.W = static_cast<int>(s->width);
  a.c = s->c;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (s->io_dtype == RGLRU_IO_F32) return dispatch_fwd<F32>(g.T, V, a, st);
  return dispatch_fwd<BF16>(g.T, V, a, st);
}

rglru_status_t rglru_bwd(const rglru_shape_t* s, const void* x, const void* gate_x, const void* gate_a,
                         const float* lambda, const uint8_t* reset, const float* ckpt, const void* dh,
                         const float* dh_last, void* dx, void* dgate_x, void* dgate_a, float* dlambda,
                         float* dh0, void* workspace, size_t workspace_bytes, void* stream) {
  if (!shape_ok(s)) return RGLRU_ERR_INVALID_ARGUMENT;
  if (!x || !gate_x || !gate_a || !lambda || !ckpt || !dh || !dx || !dgate_x || !dgate_a || !dlambda ||
      !workspace) {
    return RGLRU_ERR_INVALID_ARGUMENT;
  }
  const Geometry g = geometry(s);
  if (!io_aligned(x, g.io_bytes) || !io_aligned(gate_x, g.io_bytes) || !io_aligned(gate_a, g.io_bytes) ||
      !io_aligned(dh, g.io_bytes) || !io_aligned(dx, g.io_bytes) || !io_aligned(dgate_x, g.io_bytes) ||
      !io_aligned(dgate_a, g.io_bytes) || !f32_aligned(lambda) || !f32_aligned(ckpt) ||
      !f32_aligned(dh_last) || !f32_aligned(dlambda) || !f32_aligned(dh0) || !aligned_to(workspace, 256)) {
    return RGLRU_ERR_MISALIGNED;
  }
  if (workspace_bytes < bwd_ws(s)) return RGLRU_ERR_WORKSPACE_TOO_SMALL;

  const int V = pick_vec(RGLRU_BWD_VMAX, s->width, g.io_bytes, {x, gate_x, gate_a, dh, dx, dgate_x, dgate_a},
                         {ckpt, dh_last, dh0});
  const Slots sl = slots_in(workspace, slot_words(s, g.n_chunks_b));
  BwdArgs a;
  a.x = x;
  a.gx = gate_x;
  a.ga = gate_a;
  a.lam = lambda;
  a.reset = reset;
  a.ckpt = ckpt;
  a.dh = dh;
  a.dh_last = dh_last;
  a.dx = dx;
  a.dgx = dgate_x;
  a.dga = dgate_a;
  a.dlam = dlambda;
  a.dh0 = dh0;
  a.hdr = sl.hdr;
  a.slot_a = sl.a;
  a.slot_b = sl.b;
  a.slot_h = sl.h;
  a.slot_p = sl.p;
  a.L = s->length;
  a.n_ckpt = g.n_ckpt;
  a.B = static_cast<int>(s->batch);
  a.W = static_cast<int>(s->width);
  a.c = s->c;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (s->io_dtype == RGLRU_IO_F32) return dispatch_bwd<F32>(g.Tb, V, a, st);
  return dispatch_bwd<BF16>(g.Tb, V, a, st);
}

const char* rglru_status_string(rglru_status_t status) {
  switch (status) {
    case RGLRU_OK: return "RGLRU_OK";
    case RGLRU_ERR_INVALID_ARGUMENT: return "RGLRU_ERR_INVALID_ARGUMENT: bad shape, NULL required pointer or bad enum";
    case RGLRU_ERR_MISALIGNED: return "RGLRU_ERR_MISALIGNED: a pointer is not aligned to its element size";
    case RGLRU_ERR_WORKSPACE_TOO_SMALL: return "RGLRU_ERR_WORKSPACE_TOO_SMALL";
    case RGLRU_ERR_UNSUPPORTED: return "RGLRU_ERR_UNSUPPORTED: valid request not implemented in this build";
    case RGLRU_ERR_HIP: return "RGLRU_ERR_HIP: the HIP runtime refused a launch";
  }
  return "RGLRU_ERR_UNKNOWN";
}

int rglru_abi_version(void) { return RGLRU_ABI_VERSION; }

}  // extern "C"
