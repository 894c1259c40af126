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
// taken in chunk order from an atomic ticket, so every tile a workgroup waits
// on belongs to a workgroup that is running or done.
#include <hip/hip_runtime.h>

#include <cstring>
#include <stddef.h>
#include <stdint.h>
#include <math.h>

#include <atomic>
#include <initializer_list>
#include <mutex>
#include <type_traits>

#include "common.h"

namespace rglru {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kCkpt = RGLRU_CKPT_STEPS;
// Segment word of a token of packed sequences: the segment's index in the low
// 30 bits, bit 30 set on its first token, bit 31 on its last.
constexpr uint32_t kSegId = 0x3FFFFFFFu;
constexpr uint32_t kSegStart = 1u << 30;
constexpr uint32_t kSegEnd = 1u << 31;
constexpr unsigned kSpinLimit = 1u << 20;
// Sleep between polls (units of 64 clocks). The load and control waves share
// their SIMDs with data waves and poll at high priority, so they poll less
// often: their waits have an iteration of slack. The data waves' waits are on
// the critical path and poll at the shortest interval.
constexpr int kHelperSleep = 8;
constexpr int kLookBackSleep = 4;
constexpr size_t kHeaderBytes = 256;
constexpr int kMaxStrip = 512;   // widest channel strip of any variant (64 lanes * 8)

// Widest vector (channels per lane) the forward and backward may use; the
// host picks the widest one that divides W and matches the pointers' alignment.
#ifndef RGLRU_FWD_LOOKBACK
#define RGLRU_FWD_LOOKBACK 4
#endif
#ifndef RGLRU_FWD_VMAX
#define RGLRU_FWD_VMAX 4
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
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

template <int BYTES> struct Raw;
template <> struct Raw<2> { using T = uint16_t; };
template <> struct Raw<4> { using T = uint32_t; };
template <> struct Raw<8> { using T = u32x2; };
template <> struct Raw<16> { using T = u32x4; };

// A wave-uniform pointer, forced into scalar registers and the global
// address space, so that accesses at base + 32-bit per-lane byte offset use
// the scalar-base address form (one VGPR per lane instead of a 64-bit pair).
typedef __attribute__((address_space(1))) const char gbyte;
typedef __attribute__((address_space(1))) char gbyte_w;

__device__ __forceinline__ uint64_t uniform_u64(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ gbyte* uniform_gptr(const void* p) {
  return reinterpret_cast<gbyte*>(uniform_u64(reinterpret_cast<uint64_t>(p)));
}

__device__ __forceinline__ gbyte_w* uniform_gptr_w(void* p) {
  return reinterpret_cast<gbyte_w*>(uniform_u64(reinterpret_cast<uint64_t>(p)));
}

// 16 bytes per lane from global memory straight into LDS: lane l writes
// dst + 16 * l. The 16-byte form exists only on gfx950, so the host pass
// (which checks builtins against its own target) does not see it.
__device__ __forceinline__ void lds_dma16(gbyte* src, void* dst) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(const_cast<gbyte_w*>(src), dst, 16, 0, 0);
#endif
}

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
  // streaming (read-once / write-once) accesses at a wave-uniform base plus a
  // 32-bit per-lane element offset (selects the scalar-base address form)
  static __device__ __forceinline__ R load_nt32(const elem* base, unsigned off) {
    const gbyte* b = uniform_gptr(base);
    return __builtin_nontemporal_load(
        reinterpret_cast<__attribute__((address_space(1))) const R*>(b + off * static_cast<unsigned>(sizeof(elem))));
  }
  static __device__ __forceinline__ void store_nt32(elem* base, unsigned off, R r) {
    gbyte_w* b = uniform_gptr_w(base);
    __builtin_nontemporal_store(
        r, reinterpret_cast<__attribute__((address_space(1))) R*>(b + off * static_cast<unsigned>(sizeof(elem))));
  }
  static __device__ __forceinline__ R load_nt(const void* base, long long off) {
    return __builtin_nontemporal_load(reinterpret_cast<const R*>(reinterpret_cast<const elem*>(base) + off));
  }
  static __device__ __forceinline__ void store_nt(void* base, long long off, R r) {
    __builtin_nontemporal_store(r, reinterpret_cast<R*>(reinterpret_cast<elem*>(base) + off));
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

// 1 - 2^y for y <= 0, given a = 2^y. For y > log2 0.9 (a > 0.9, where 1 - a
// would cancel) it is -y * q(y) with q a cubic approximation of
// -expm1(y ln 2) / (-y): the interpolant at the four Chebyshev nodes of
// [log2 0.9, 0], within 8e-9 relative of it there (a quartic Taylor series
// in y ln 2 is within 2e-8 and costs one more fma). Elsewhere 1 - a >= 0.1,
// so the rounding of a costs at most about 1e-6 relative. The stationary
// factor sqrt(1 - a^2) thus keeps float32 precision when a is close to 1.
__device__ __forceinline__ float one_minus_exp2(float y, float a) {
  float q = 0.00922239626706585f;
  q = fmaf(q, y, 0.05546679335497464f);
  q = fmaf(q, y, 0.24022537591902696f);
  q = fmaf(q, y, 0.6931471751903574f);
  const float near0 = -y * q;
  return (y > -0.15200309f) ? near0 : 1.0f - a;
}

// softplus(lambda) = max(lambda, 0) + log1p(e^-|lambda|) on the hardware exp2
// and log2. log1p(z) uses Kahan's formulation, ln(1 + z) * z / ((1 + z) - 1),
// which cancels the rounding of 1 + z (Goldberg, "What Every Computer
// Scientist Should Know About Floating-Point Arithmetic", 1991, Theorem 4: a
// few ulp), and z itself where 1 + z rounds to 1. About a third of the
// instructions of the library expf and log1pf, which the load wave runs for
// every tile.
__device__ __forceinline__ float softplus_f(float lam) {
  const float z = __builtin_amdgcn_exp2f(-kLog2e * fabsf(lam));
  const float u = 1.0f + z;
  const float d = u - 1.0f;
  const float l1p = d == 0.0f ? z : __builtin_amdgcn_logf(u) * (0.69314718f * z) * __builtin_amdgcn_rcpf(d);
  return fmaxf(lam, 0.0f) + l1p;
}

// Per-channel decay constants: cs = -c * softplus(lambda), k2 = cs * log2 e.
__device__ __forceinline__ void channel_consts(float lam, float c, float& cs, float& k2) {
  cs = -c * softplus_f(lam);
  k2 = cs * kLog2e;
}

// ------------------------------------------------------------------ look-back slots

__device__ __forceinline__ void publish(u64* slot, size_t idx, unsigned tag, uint32_t bits) {
  const u64 w = (static_cast<u64>(tag) << 32) | static_cast<u64>(bits);
  __hip_atomic_store(slot + idx, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// poll at a wave-uniform slot pointer plus a per-lane byte offset
__device__ __forceinline__ u64 poll_at(const u64* uniform_slot, unsigned lane_bytes) {
  gbyte* b = uniform_gptr(uniform_slot);
  return __hip_atomic_load(reinterpret_cast<__attribute__((address_space(1))) const u64*>(b + lane_bytes),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

// The high half of Header::counter counts calls; a forward tags the words it
// publishes with that count + 1. The backward's words carry 0 in their high
// half, so the count skips 0xFFFFFFFF: every tag lies in [1, 0xFFFFFFFF] and
// repeats only after 2^32 - 1 calls. Run by the last workgroup of a call,
// when no other workgroup of the call touches the header: the next call
// starts with no tickets handed out.
__device__ __forceinline__ void advance_call(Header* hdr) {
  const u64 c = __hip_atomic_load(&hdr->counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  unsigned next = static_cast<unsigned>(c >> 32) + 1u;
  if (next == 0xFFFFFFFFu) next = 0u;
  __hip_atomic_store(&hdr->counter, static_cast<u64>(next) << 32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Carry entering a tile, computed by one wave (a control wave), one channel
// per lane. A round polls the published words of the K nearest predecessors
// (tiles of earlier chunks of the same row in the forward, later chunks in the
// backward) in one memory round trip, finds the nearest one whose outgoing
// carry is known (published, fixed by a reset inside it, or the sequence
// start) with every map between published, and applies those maps oldest
// first with the very fma the predecessors use for their own outgoing
// carries: the carry is bit-identical to the serial chain whatever the timing
// (deterministic). `self` is the slot index of the lane's channel, split into
// a wave-uniform part and the lane (the polls address a scalar base plus one
// 32-bit lane offset); `stride` is the slot distance between consecutive
// predecessors, `npred` how many exist. Returns whether this lane's carry was
// found (it is then in `carry`).
template <int K, bool EARLY_OUT>
__device__ __forceinline__ bool look_back_round(const u64* slot_a, const u64* slot_b, const u64* slot_h,
                                                long long self_uniform, unsigned lane, long long stride, int npred,
                                                unsigned tag, float init, float& carry) {
  const unsigned lane_bytes = lane * 8u;
  u64 wh[K], wa[K], wb[K];
  if constexpr (!EARLY_OUT) {
    // the nearest predecessor's published carry first: once every channel
    // of the strip has it, the round needs none of the other words
    if (npred > 0) {
      const u64 h1 = poll_at(slot_h + (self_uniform - stride), lane_bytes);
      if (__builtin_amdgcn_ballot_w64(!tagged(h1, tag)) == 0ull) {
        carry = __uint_as_float(static_cast<uint32_t>(h1));
        return true;
      }
    }
#pragma unroll
    for (int d = 0; d < K; ++d) {
      const long long q = self_uniform - static_cast<long long>(d + 1) * stride;
      wh[d] = d < npred ? poll_at(slot_h + q, lane_bytes) : 0ull;
      wa[d] = d < npred ? poll_at(slot_a + q, lane_bytes) : 0ull;
      wb[d] = d < npred ? poll_at(slot_b + q, lane_bytes) : 0ull;
    }
  } else {
    // The same first poll; then, without the nearest predecessor's carry and
    // map no channel can get further this round, so the farther words are
    // read only when some channel has that map (fewer words polled, one more
    // round trip when the map is there but the carry is not).
    if (npred > 0) {
      const long long q0 = self_uniform - stride;
      wh[0] = poll_at(slot_h + q0, lane_bytes);
      if (__builtin_amdgcn_ballot_w64(!tagged(wh[0], tag)) == 0ull) {
        carry = __uint_as_float(static_cast<uint32_t>(wh[0]));
        return true;
      }
      wa[0] = poll_at(slot_a + q0, lane_bytes);
      wb[0] = poll_at(slot_b + q0, lane_bytes);
      const bool stuck = !tagged(wh[0], tag) && !(tagged(wa[0], tag) && tagged(wb[0], tag));
      if (__builtin_amdgcn_ballot_w64(!stuck) == 0ull) return false;
    } else {
      wh[0] = wa[0] = wb[0] = 0ull;
    }
#pragma unroll
    for (int d = 1; d < K; ++d) {
      const long long q = self_uniform - static_cast<long long>(d + 1) * stride;
      wh[d] = d < npred ? poll_at(slot_h + q, lane_bytes) : 0ull;
      wa[d] = d < npred ? poll_at(slot_a + q, lane_bytes) : 0ull;
      wb[d] = d < npred ? poll_at(slot_b + q, lane_bytes) : 0ull;
    }
  }
  int start = -1;
  int kind = 0;     // 1: published carry, 2: map with a reset, 3: sequence start
  bool open = true; // every nearer map is published
#pragma unroll
  for (int d = 0; d < K; ++d) {
    if (open && start < 0) {
      if (d >= npred) {
        start = d;
        kind = 3;
      } else if (tagged(wh[d], tag)) {
        start = d;
        kind = 1;
      } else if (!(tagged(wa[d], tag) && tagged(wb[d], tag))) {
        open = false;
      } else if ((static_cast<uint32_t>(wa[d]) >> 31) != 0) {
        start = d;
        kind = 2;
      }
    }
  }
  if (start < 0) return false;
  float hv = 0.0f;
  bool have = false;
#pragma unroll
  for (int d = K - 1; d >= 0; --d) {
    const float hd = __uint_as_float(static_cast<uint32_t>(wh[d]));
    const float ad = __uint_as_float(static_cast<uint32_t>(wa[d]) & 0x7FFFFFFFu);
    const float bd = __uint_as_float(static_cast<uint32_t>(wb[d]));
    if (d == start) {
      hv = kind == 1 ? hd : (kind == 2 ? bd : init);
      have = true;
    } else if (have) {
      hv = fmaf(ad, hv, bd);
    }
  }
  carry = hv;
  return true;
}

// Rounds until the carry is found; false if the spin limit was reached (the
// carry is then 0).
template <int K, bool EARLY_OUT>
__device__ __forceinline__ bool look_back_wave(const u64* slot_a, const u64* slot_b, const u64* slot_h,
                                               long long self_uniform, unsigned lane, long long stride, int npred,
                                               unsigned tag, float init, float& carry) {
  for (unsigned round = 0; round < kSpinLimit; ++round) {
    if (look_back_round<K, EARLY_OUT>(slot_a, slot_b, slot_h, self_uniform, lane, stride, npred, tag, init, carry)) {
      return true;
    }
    __builtin_amdgcn_s_sleep(kLookBackSleep);
  }
  carry = 0.0f;
  return false;
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
  // packed sequences (batch row 0 only; nullptr otherwise): per-token
  // segment word (segment id, start and end bits), the segments' initial and
  // final states [n_segments, W]
  const uint32_t* seg;
  const float* h0s;
  float* h_last_s;
  // gate projections computed inside the forward (256-wide blocks): the
  // weights of each gate in MFMA fragment order (one 1 KiB fragment per
  // block, 32-output tile and 16-input step), the biases [W] bf16 (or
  // nullptr), and where the logits also go [B*L, W] (or nullptr)
  const uint16_t* wt[2];
  const uint16_t* pbias[2];
  uint16_t* gout[2];
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
  bool h_wide;           // h rows start 16-byte aligned (W * sizeof(io) % 16 == 0, h aligned)
};

// Flags in LDS between the waves of a workgroup: workgroup-scope relaxed
// atomics on the LDS word itself, which compile to plain ds_write / ds_read
// (no wait on the issuing wave's global memory traffic). A writer makes its
// data visible first (lds_release: its LDS operations have completed, and the
// compiler keeps them before the flag); a reader keeps its data reads after
// the flag (lds_acquire).
__device__ __forceinline__ int lds_load(const int* f) {
  return __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_store(int* f, int v) {
  __hip_atomic_store(f, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_add(int* f, int v) {
  __hip_atomic_fetch_add(f, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_release() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void lds_acquire() { asm volatile("" ::: "memory"); }

// Bounded wait for an LDS word to reach v (EQ: equal; otherwise at least v).
// A wait that reaches the spin limit sets bit 1 of the sticky error word and
// the workgroup's abort word; once that is set every wait returns at once, so
// the workgroup always drains and exits (the call's outputs are then invalid,
// as the error word says).
template <bool EQ, int SLEEP = 1>
__device__ __forceinline__ void lds_wait(const int* f, int v, int* abort, Header* hdr) {
  for (unsigned n = 0; n < kSpinLimit; ++n) {
    const int c = lds_load(f);
    if (EQ ? c == v : c >= v) {
      lds_acquire();
      return;
    }
    if (lds_load(abort) != 0) return;
    __builtin_amdgcn_s_sleep(SLEEP);
  }
  lds_store(abort, 1);
  if ((threadIdx.x & 63) == 0) atomicOr(&hdr->err, 2u);
}

// s_waitcnt immediates (gfx9 layout: vmcnt[3:0] and [15:14], expcnt[6:4], lgkmcnt[11:8])
constexpr int kWaitVm0 = 0x0F70;    // vmcnt(0), other counters unconstrained

// Fused projection helpers. A pass works on one gate and one 32-output tile
// (outputs sub*64 + op*32 + lane%32 of block kb) with
// v_mfma_f32_32x32x16_bf16 (A 32x16, B 16x32; lane l holds row/column l%32
// and k = (l/32)*8 .. +7; D lane l holds column l%32, register r row
// (r/4)*8 + (l/32)*4 + r%4): its weights are the A operands of the 16 input
// steps of 16. The call lays them out beforehand in fragment order, so that
// each is one contiguous 1 KiB load: fragment (kb, ot, ks) holds, for lane l,
// inputs ks*16 + (l/32)*8 .. +7 of output ot*32 + l%32.
__device__ __forceinline__ bf16x8 fused_w_frag(const uint16_t* wf, int kb, int sub, int op, int ks, int lane) {
  const long long frag = (static_cast<long long>(kb) * 8 + sub * 2 + op) * 16 + ks;
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(wf + (frag * 64 + lane) * 8));
}

// LDS reads of the token operands, issued as inline assembly so that they
// stay the written distance ahead of their MFMAs (compiled reads are placed
// one step ahead). fused_lds_wait waits until at most N LDS operations of the
// wave are outstanding (they complete in order) and ties the two values read,
// so that no use of them moves above it.
__device__ __forceinline__ uint32_t lds_off(const void* ptr) {
  typedef __attribute__((address_space(3))) const char lds_char;
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_char*)(ptr)));
}
template <int OFF = 0>
__device__ __forceinline__ u32x4 fused_lds_read16(uint32_t addr) {
  u32x4 d;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(d) : "v"(addr), "n"(OFF));
  return d;
}
constexpr int kFusedAhead = 1;   // input steps of token operands read ahead
template <int N>
__device__ __forceinline__ void fused_lds_wait(u32x4& x, u32x4& y) {
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(x), "+v"(y) : "n"(N));
}

// Persistent, software-pipelined forward.
//
// A tile is one batch row b, a strip of 64 channels (one channel per lane) and
// T = NW * TS steps. Tiles are handed out in chunk order by an atomic ticket,
// so every tile a look-back waits on belongs to a workgroup that is running or
// done. A workgroup has NW data waves (wave w owns steps w*TS .. w*TS+TS-1 of
// every tile), two control waves and two load waves; there is no barrier
// inside the pipeline, only one-directional LDS flags. With t_i the
// workgroup's i-th tile:
//   load wave i%2    : once every data wave has finished with LDS buffer i%2
//                      (tile t_{i-2}), streams the raw words of t_i (x, gate_x,
//                      gate_a and the reset flags) from HBM into it with
//                      global_load_lds and evaluates the tile's decay
//                      constants, so two tiles of loads are in flight while
//                      the data waves compute a third. Load wave 0 draws the
//                      tickets, two at a time and two iterations ahead, so a
//                      workgroup's tiles come in ticket order;
//   data waves       : in iteration i, evaluate the gates of t_i as (alpha,
//                      write) pairs, reduce their steps to an affine map
//                      h -> R ? B : A*h + B and report it, and in the same
//                      straight-line block replay t_{i-2} from the pairs kept
//                      since then (a ring of three tiles in registers) and its
//                      incoming carry, storing h and the checkpoint. The
//                      replay's serial fma chain hides in the gate arithmetic,
//                      and the carry of t_{i-2} has had a whole iteration to
//                      arrive;
//   control wave i%2 : once every data wave has reported t_i, writes the
//                      per-wave prefix maps the replay starts from, publishes
//                      the tile's map, runs its look-back, publishes its
//                      outgoing carry and hands the incoming one to the data
//                      waves. Two control waves give each tile's publish and
//                      look-back two iterations.
// The data waves issue no global loads and the control waves only their
// polls, so no wave waits behind memory traffic it does not need (the vector
// memory counter retires in order).
//
// LDS rows: WIDE loads move 16 bytes per lane, so one instruction fills 1 KiB
// of consecutive step rows (8 rows of 64 bf16 channels, 4 of 64 float32); a
// row in LDS is then 64 * sizeof(io) bytes. Otherwise each instruction fills
// one row with 2 or 4 bytes per lane, each lane's value zero-extended into its
// own 4-byte slot (rows of 256 bytes).
template <typename IO, int NW, int TS, bool WIDE, bool PACKED, bool FUSED>
__global__ __launch_bounds__((NW + (FUSED ? 8 : 4)) * 64) void fwd_kernel(FwdArgs p) {
  using elem = typename IO::elem;
  using io = Io<IO, 1>;
  constexpr bool BF = std::is_same<IO, BF16>::value;
  constexpr int ES = static_cast<int>(sizeof(elem));
  constexpr int T = NW * TS;
  constexpr int ROWB = WIDE ? 64 * ES : 256;
  constexpr int SEG = ROWB / 16;           // 16-byte segments per row (WIDE)
  constexpr int RPI = 64 / SEG;            // rows per 16-byte-per-lane instruction (WIDE)
  constexpr int K = RGLRU_FWD_LOOKBACK;
  constexpr int RING = 16;
  constexpr int NFL = T < 64 ? 64 : T;     // reset-flag slots per buffer (one instruction fills 64)
  constexpr int CTRL0 = NW, LOAD0 = NW + 2, PROJ0 = NW + 4;
  static_assert(TS % kCkpt == 0, "checkpoints fall on wave boundaries, at compile-time steps of a wave");
  static_assert(TS <= 16 && NW <= 32, "a wave's cut and end flags share one mask word; the waves' flags fit one");
  static_assert(!WIDE || T % RPI == 0, "a tile is a whole number of 16-byte-per-lane instructions");
  static_assert(NFL % 64 == 0 && NFL <= 128, "reset flags: at most two instructions");
  static_assert(!FUSED || (std::is_same<IO, BF16>::value && WIDE && T == 64 && TS == 8 && !PACKED),
                "the fused projection runs bf16 tiles of two 32-token MFMA tiles");

  __shared__ __attribute__((aligned(16))) unsigned char s_raw[2][3][T][ROWB];
  // fused projection: the tile's rows of x across its whole 256-wide block
  // (16-byte granules XOR-swizzled by row, so the MFMA operand reads of 16
  // rows fall on distinct banks)
  __shared__ __attribute__((aligned(16))) uint16_t s_xb[FUSED ? 2 : 1][FUSED ? T : 1][256];
  __shared__ unsigned s_rflag[2][NFL];
  __shared__ uint32_t s_seg[2][NFL];  // segment words (packed sequences)
  __shared__ uint32_t s_endseg[3][NW][TS];   // a wave's segment ends, per ring slot
  __shared__ float s_k2[2][64];
  // per map slot (iteration % 3): the data waves' maps, the prefixes the
  // replay starts from and the tile's incoming carry
  __shared__ float s_A[3][NW][64];
  __shared__ float s_B[3][NW][64];
  __shared__ unsigned s_R[3][NW];
  __shared__ float s_PA[3][NW][64];   // composite of the maps of the waves before each wave
  __shared__ float s_PB[3][NW][64];
  __shared__ unsigned s_PRm[3];       // bit w: a reset inside the waves before wave w
  __shared__ float s_carry[3][64];
  __shared__ __attribute__((aligned(16))) elem s_hst[NW][TS * 64];   // a wave's h rows, staged for 16-byte stores
  __shared__ unsigned s_tk[RING];     // tile of iteration i in s_tk[i % RING]
  __shared__ unsigned s_tag;
  __shared__ int s_tk_valid;          // highest iteration whose ticket is in s_tk
  __shared__ int s_full[2];           // iteration whose raw words buffer j holds
  __shared__ int s_cons[2];           // data waves done with buffer j so far
  __shared__ int s_maps_in[3];        // data-wave maps reported for iterations of each slot so far
  __shared__ int s_carry_ok[3];       // iteration whose incoming carry slot s holds
  __shared__ int s_prog[NW];          // iteration each data wave is in
  __shared__ __attribute__((aligned(16))) float s_fbias[FUSED ? 2 : 1][2][64];   // fused: the strip's biases per gate
  __shared__ int s_xb_full[2];        // fused: iteration whose block rows s_xb[j] holds
  __shared__ int s_proj_done[2];      // fused: projection passes finished on buffer j so far
  __shared__ int s_abort;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const unsigned rows = static_cast<unsigned>(p.B) * static_cast<unsigned>(p.n_strips);
  const long long W = p.W;

  if (threadIdx.x == 0) {
    s_tk_valid = -1;
    s_full[0] = s_full[1] = -1;
    s_xb_full[0] = s_xb_full[1] = -1;
    s_proj_done[0] = s_proj_done[1] = 0;
    s_cons[0] = s_cons[1] = 0;
    s_maps_in[0] = s_maps_in[1] = s_maps_in[2] = 0;
    s_carry_ok[0] = s_carry_ok[1] = s_carry_ok[2] = -1;
#pragma unroll
    for (int w = 0; w < NW; ++w) s_prog[w] = -1;
    s_abort = 0;
  }
  __syncthreads();

  struct Tile {
    bool valid, active;
    int chunk, b, strip, ch;
    long long t0, rowbase;
  };
  // Lambdas capture by value: a by-reference capture of the kernel arguments
  // takes their address and moves them to scratch memory.
  auto tile_of = [=](unsigned tile) {
    Tile t;
    t.valid = tile < p.n_tiles;
    const unsigned tt = t.valid ? tile : 0u;
    t.chunk = static_cast<int>(tt / rows);
    const int row = static_cast<int>(tt - static_cast<unsigned>(t.chunk) * rows);
    t.b = row / p.n_strips;
    t.strip = row - t.b * p.n_strips;
    t.ch = t.strip * 64 + lane;
    t.active = t.ch < p.W;
    t.t0 = static_cast<long long>(t.chunk) * T;
    t.rowbase = static_cast<long long>(t.b) * p.L;
    return t;
  };
  auto ticket_tile = [=](u64 v, unsigned m) {
    const unsigned q = static_cast<unsigned>(v) + m;
    return q < p.n_tiles ? q : p.n_tiles;
  };
  // Both gate projections of tile t from its block rows in s_xb[jb], into the
  // gate_x and gate_a rows of raw buffer jb (bf16, rounded once) and, when
  // asked, to the logit outputs: gate_g = x[:, blk] w_g[blk] + b_g[blk] as
  // D = w_g^T x^T on v_mfma_f32_16x16x32_bf16 (A: lane l holds output l%16,
  // inputs (l/16)*8 .. +7 of a 32-input step; B: token l%16, the same inputs;
  // D: token l%16, outputs (l/16)*4 .. +3), accumulators started at the bias
  // and the eight input steps in order, as the projection kernel does, so
  // the logits are bitwise those of rglru_blockdiag_gate_proj_fwd.
  //
  // Work of one pass: one gate, two 16-output tiles (weights in registers)
  // against two 16-token tiles at a time, so four independent accumulator
  // chains hide the MFMA latency and each token operand read from LDS feeds
  // two products. A pass's weights come from the pre-transposed copy
  // ([out][in], L2-resident: every tile of a strip reads the same 64 KiB).
  // The gate rows the passes write are swizzled: 8-byte chunk c of row r
  // (channels 4c .. 4c+3) sits at chunk c ^ ((r >> 1) & 15), so that the 32
  // rows one write instruction covers fall on distinct banks; the data waves
  // read them through the same map.
  //
  // a holds the pass's weights; the biases come from s_fbias[jb][g].
  auto project_pass = [=](int jb, const Tile& t, long long lim, int g, int op, const bf16x8 (&a)[16]) {
    if constexpr (FUSED) {
      const int kb = t.strip >> 2;
      const int sub = t.strip & 3;
      const int lr = lane & 31;
      const int hi = lane >> 5;
      // token operand of input step ks, token tile tp: row tp*32 + lr, source
      // granule ks*2 + hi, stored at granule (ks*2 + hi) ^ (lr % 16); the
      // swizzle acts on the offset within the buffer, which starts at xbase
      const uint32_t xbase = lds_off(&s_xb[jb][0][0]);
      // (from a lane index opaque here, so that the read addresses are formed
      // as they are used instead of being kept in registers across tiles)
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const uint32_t xrow = static_cast<uint32_t>((ln & 31) * 512 + (((ln >> 5) ^ (ln & 15)) << 4));
      // token tile 1 is 32 rows (16 KiB) further: an immediate offset
      auto xread = [&](int ks, u32x4 (&dst)[2]) {
        const uint32_t ad = xbase + (xrow ^ static_cast<uint32_t>(ks << 5));
        dst[0] = fused_lds_read16<0>(ad);
        dst[1] = fused_lds_read16<32 * 512>(ad);
      };
      f32x16 acc[2];   // [token tile]
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 b4 = *reinterpret_cast<const f32x4*>(&s_fbias[jb][g][op * 32 + j * 8 + hi * 4]);
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[0][j * 4 + q] = acc[1][j * 4 + q] = b4[q];
      }
      u32x4 xv[16][2];
#pragma unroll
      for (int ks = 0; ks < kFusedAhead; ++ks) xread(ks, xv[ks]);
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) {
        // in flight: steps ks .. min(ks + kFusedAhead - 1, 15), two reads each
        constexpr int kLast = 16 - kFusedAhead;
        if (ks <= kLast) {
          fused_lds_wait<2 * (kFusedAhead - 1)>(xv[ks][0], xv[ks][1]);
        } else {
          fused_lds_wait<0>(xv[ks][0], xv[ks][1]);
        }
        if (ks + kFusedAhead < 16) xread(ks + kFusedAhead, xv[ks + kFusedAhead]);
#pragma unroll
        for (int v = 0; v < 2; ++v) {
          acc[v] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks], __builtin_bit_cast(bf16x8, xv[ks][v]), acc[v], 0, 0,
                                                           0);
        }
      }
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        const int tr = v * 32 + lr;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint2 w2;
          w2.x = f32x2_to_bf16x2(acc[v][j * 4 + 0], acc[v][j * 4 + 1]);
          w2.y = f32x2_to_bf16x2(acc[v][j * 4 + 2], acc[v][j * 4 + 3]);
          *reinterpret_cast<uint2*>(&s_raw[jb][1 + g][tr][((op * 8 + j * 2 + hi) ^ ((tr >> 1) & 15)) * 8]) = w2;
        }
      }
    }
  };

  if (FUSED && wave >= PROJ0) {
    // ------------------------------------------------------------ projection waves
    // Wave PROJ0 + q computes pass q of every tile: gate q / 2, outputs
    // (q % 2) * 32 .. +31 of the strip, once the tile's block rows have
    // landed and its raw buffer is free (s_xb_full), and counts it done.
    if constexpr (FUSED) {
      __builtin_amdgcn_s_setprio(3);
      const int q = wave - PROJ0;
      const int g = q >> 1, op = q & 1;
      const uint16_t* wf = g ? p.wt[1] : p.wt[0];
      for (int i = 0;; ++i) {
        lds_wait<false, kHelperSleep>(&s_tk_valid, i, &s_abort, p.hdr);
        if (lds_load(&s_abort) != 0) break;
        const unsigned tile = __builtin_amdgcn_readfirstlane(s_tk[i % RING]);
        if (tile >= p.n_tiles) break;
        const Tile t = tile_of(tile);
        const int jb = i & 1;
        const int kb = t.strip >> 2, sub = t.strip & 3;
        // this pass's weights (L2-resident) while the rows land
        bf16x8 a[16];
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) a[ks] = fused_w_frag(wf, kb, sub, op, ks, lane);
        lds_wait<false, kHelperSleep>(&s_xb_full[jb], i, &s_abort, p.hdr);
        if (lds_load(&s_abort) != 0) break;
        project_pass(jb, t, p.L - 1 - t.t0, g, op, a);
        lds_release();
        if (lane == 0) lds_add(&s_proj_done[jb], 1);
      }
    }
  } else if (wave >= LOAD0) {
    // ------------------------------------------------------------ load waves
    __builtin_amdgcn_s_setprio(3);
    const int j = wave - LOAD0;
    if (j == 0) {
      u64 v = 0;
      if (lane == 0) v = atomicAdd(&p.hdr->counter, 2ull);
      v = uniform_u64(v);
      if (lane == 0) {
        s_tk[0] = ticket_tile(v, 0);
        s_tk[1] = ticket_tile(v, 1);
        s_tag = static_cast<unsigned>(v >> 32) + 1u;
      }
      lds_release();
      if (lane == 0) lds_store(&s_tk_valid, 1);
    }
    const unsigned char* src[3] = {static_cast<const unsigned char*>(p.x), static_cast<const unsigned char*>(p.gx),
                                   static_cast<const unsigned char*>(p.ga)};
    const long long row_bytes = W * ES;
    for (int i = j;; i += 2) {
      lds_wait<false, kHelperSleep>(&s_tk_valid, i, &s_abort, p.hdr);
      const Tile t = tile_of(__builtin_amdgcn_readfirstlane(s_tk[i % RING]));
      const long long lim = p.L - 1 - t.t0;   // last step row of the tile inside the sequence
      if constexpr (FUSED) {
        // The tile's rows across its whole block go to this wave's own block
        // buffer, free once the projection waves are done with tile t_{i-2},
        // so they are in flight before the raw buffer is: 2 rows of 512 bytes
        // per instruction, lane l at row l / 32, LDS granule l % 32, which
        // holds source granule (l % 32) ^ (row % 16).
        lds_wait<false, kHelperSleep>(&s_proj_done[j], 4 * (i / 2), &s_abort, p.hdr);
        if (t.valid && lds_load(&s_abort) == 0) {
          const int kb = t.strip >> 2;
          gbyte* base = uniform_gptr(static_cast<const unsigned char*>(p.x) + (t.rowbase + t.t0) * row_bytes +
                                     static_cast<long long>(kb) * 512);
          const int rr = lane >> 5;
          const int gq = lane & 31;
#pragma unroll 4
          for (int g = 0; g < T / 2; ++g) {
            const long long row = 2 * g + rr;
            const long long rw = row < lim ? row : lim;
            const unsigned off = static_cast<unsigned>(rw) * static_cast<unsigned>(row_bytes) +
                                 static_cast<unsigned>((gq ^ (static_cast<int>(row) & 15)) * 16);
            lds_dma16(base + off, &s_xb[j][2 * g][0]);
          }
        }
      }
      // buffer j is free once every data wave is done with iteration i - 2
      lds_wait<false, kHelperSleep>(&s_cons[j], NW * (i / 2), &s_abort, p.hdr);
      if (lds_load(&s_abort) != 0) {
        __builtin_amdgcn_s_waitcnt(kWaitVm0);   // no LDS-bound load outlives the wave
        break;
      }
      if (!t.valid) {
        if (lane == 0) lds_store(&s_full[j], i);
        break;
      }
      const float lam = t.active ? p.lam[t.ch] : 0.0f;
      const long long strip_b = static_cast<long long>(t.strip) * 64 * ES;
      const long long tile_off = (t.rowbase + t.t0) * row_bytes + strip_b;
      if constexpr (WIDE) {
        // lane l: row l / SEG of each group of RPI rows, bytes (l % SEG) * 16
        // .. +15 of it. Segments past W (last strip only) re-read the strip's
        // first segment and rows past L re-read row L - 1; those words are
        // never used, so every source address stays in bounds.
        const int r = lane / SEG;
        const unsigned seg = static_cast<unsigned>(lane % SEG) * 16u;
        const unsigned col = strip_b + seg < row_bytes ? seg : 0u;
        if (t.t0 + T <= p.L) {
          // one scalar base per input, the lane's row and segment as a 32-bit
          // offset that steps by RPI rows per instruction (the host keeps a
          // tile's rows under 2 GiB)
          const unsigned step = static_cast<unsigned>(RPI) * static_cast<unsigned>(row_bytes);
#pragma unroll
          for (int q = 0; q < (FUSED ? 0 : 3); ++q) {
            gbyte* base = uniform_gptr(src[q] + tile_off);
            unsigned off = static_cast<unsigned>(r) * static_cast<unsigned>(row_bytes) + col;
            unsigned char* dst = &s_raw[j][q][0][0];
#pragma unroll 4
            for (int g = 0; g < T / RPI; ++g) {
              lds_dma16(base + off, dst);
              off += step;
              dst += 1024;
            }
          }
        } else {
#pragma unroll
          for (int q = 0; q < (FUSED ? 0 : 3); ++q) {
            gbyte* base = uniform_gptr(src[q] + tile_off);
            for (int g = 0; g < T / RPI; ++g) {
              const long long row = g * RPI + r;
              const long long off = (row < lim ? row : lim) * row_bytes + col;
              lds_dma16(base + off, &s_raw[j][q][g * RPI][0]);
            }
          }
        }
      } else {
        const unsigned col = t.active ? static_cast<unsigned>(lane * ES) : 0u;
#pragma unroll 4
        for (int k = 0; k < T; ++k) {
          const long long row = k < lim ? k : lim;
#pragma unroll
          for (int q = 0; q < 3; ++q) {
            gbyte* base = uniform_gptr(src[q] + tile_off + row * row_bytes);
            __builtin_amdgcn_global_load_lds(const_cast<gbyte_w*>(base + col), &s_raw[j][q][k][0], ES, 0, 0);
          }
        }
      }
      if (p.reset != nullptr) {
#pragma unroll
        for (int h = 0; h < NFL / 64; ++h) {
          const long long st = h * 64 + lane;
          const long long tk = t.t0 + (st < lim ? st : lim);
          __builtin_amdgcn_global_load_lds(p.reset + t.rowbase + tk, &s_rflag[j][h * 64], 1, 0, 0);
        }
      }
      if constexpr (PACKED) {
#pragma unroll
        for (int h = 0; h < NFL / 64; ++h) {
          const long long st = h * 64 + lane;
          const long long tk = t.t0 + (st < lim ? st : lim);
          __builtin_amdgcn_global_load_lds(const_cast<uint32_t*>(p.seg) + t.rowbase + tk, &s_seg[j][h * 64], 4, 0, 0);
        }
      }
      // the next two tickets, two iterations ahead (load wave 0 draws them all,
      // so a workgroup's tiles come in ticket order)
      u64 nxt = 0;
      if (j == 0 && lane == 0) nxt = atomicAdd(&p.hdr->counter, 2ull);
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      if constexpr (FUSED) {
        // the tile's x strip, from its block rows, into the raw x rows the
        // data waves read (row r at r * 128 bytes, granule gg of the strip at
        // gg * 16)
        const int sub = t.strip & 3;
        const int gg = lane & 7;
#pragma unroll
        for (int k = 0; k < T / 8; ++k) {
          const int row = k * 8 + (lane >> 3);
          const u32x4 v = *reinterpret_cast<const u32x4*>(&s_xb[j][row][((sub * 8 + gg) ^ (row & 15)) * 8]);
          *reinterpret_cast<u32x4*>(&s_raw[j][0][row][gg * 16]) = v;
        }
        // and the strip's biases of both gates (zeros without)
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const uint16_t* bsrc = g ? p.pbias[1] : p.pbias[0];
          s_fbias[j][g][lane] = bsrc != nullptr ? bf16_bits_to_f32(bsrc[t.strip * 64 + lane]) : 0.0f;
        }
      }
      {
        float cs = 0.0f, k2 = 0.0f;
        if (t.active) channel_consts(lam, p.c, cs, k2);
        s_k2[j][lane] = k2;
      }
      if (j == 0) {
        nxt = uniform_u64(nxt);
        if (lane == 0) {
          s_tk[(i + 2) % RING] = ticket_tile(nxt, 0);
          s_tk[(i + 3) % RING] = ticket_tile(nxt, 1);
        }
      }
      lds_release();
      if constexpr (FUSED) {
        // the block rows are in and the raw buffer is free: the projection
        // waves fill its gate rows, and the tile is full once all four passes
        // are (each released its writes before counting)
        if (lane == 0) {
          if (j == 0) lds_store(&s_tk_valid, i + 3);
          lds_store(&s_xb_full[j], i);
        }
        lds_wait<false, kHelperSleep>(&s_proj_done[j], 4 * (i / 2 + 1), &s_abort, p.hdr);
        if (lane == 0) lds_store(&s_full[j], i);
      } else {
        if (lane == 0) {
          if (j == 0) lds_store(&s_tk_valid, i + 3);
          lds_store(&s_full[j], i);
        }
      }
    }
  } else if (wave >= CTRL0) {
    // ------------------------------------------------------------ control waves
    __builtin_amdgcn_s_setprio(3);
    const int c = wave - CTRL0;
    unsigned tag = 0;
    for (int i = c;; i += 2) {
      lds_wait<false, kHelperSleep>(&s_tk_valid, i, &s_abort, p.hdr);
      if (lds_load(&s_abort) != 0) break;
      if (i == c) tag = __builtin_amdgcn_readfirstlane(s_tag);
      const unsigned tile = __builtin_amdgcn_readfirstlane(s_tk[i % RING]);
      if (tile >= p.n_tiles) break;
      const int ms = i % 3;
      const Tile t = tile_of(tile);
      const size_t sidx = static_cast<size_t>(tile) * 64 + lane;
      const bool last = t.chunk == p.n_chunks - 1;
      const float init = (t.active && p.h0 != nullptr) ? p.h0[t.b * W + t.ch] : 0.0f;
      // A look-back needs only the predecessors' words, so one round goes out
      // before this tile's maps are in: its predecessors are usually far
      // enough along that the carry is known by the time the maps are, and
      // the tile then publishes its outgoing carry at once.
      float carry = init;
      bool found = true;
      if (t.active && t.chunk > 0) {
        found = look_back_round<K, false>(p.slot_a, p.slot_b, p.slot_h, static_cast<long long>(tile) * 64,
                                   static_cast<unsigned>(lane), static_cast<long long>(rows) * 64, t.chunk, tag, init,
                                   carry);
      }
      // once every data wave has reported its map of t_i: the prefixes the
      // replay starts from and the tile's map. A data wave may report up to
      // two iterations ahead of another (its replay of t_{i-2} waits for the
      // carry of t_{i-2}), so the reports are counted per slot of three.
      lds_wait<false, kHelperSleep>(&s_maps_in[ms], NW * (i / 3 + 1), &s_abort, p.hdr);
      if (lds_load(&s_abort) != 0) break;
      float Aw[NW], Bw[NW];
      unsigned Rw[NW];
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        Rw[w] = s_R[ms][w];
        Aw[w] = s_A[ms][w][lane];
        Bw[w] = s_B[ms][w][lane];
      }
      float GA = 1.0f, GB = 0.0f;
      bool GR = false;
      unsigned prbits = 0u;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        s_PA[ms][w][lane] = GA;
        s_PB[ms][w][lane] = GB;
        prbits |= GR ? (1u << w) : 0u;
        GB = Rw[w] != 0u ? Bw[w] : fmaf(Aw[w], GB, Bw[w]);
        GA *= Aw[w];
        GR = GR || Rw[w] != 0u;
      }
      if (lane == 0) s_PRm[ms] = prbits;
      // otherwise publish the map, finish the look-back; then publish the
      // outgoing carry (not needed after the last chunk)
      if (t.active) {
        if (!found) {
          if (!last) {
            publish(p.slot_a, sidx, tag, encode_a(GA, GR));
            publish(p.slot_b, sidx, tag, __float_as_uint(GB));
          }
          if (!look_back_wave<K, false>(p.slot_a, p.slot_b, p.slot_h, static_cast<long long>(tile) * 64,
                                 static_cast<unsigned>(lane), static_cast<long long>(rows) * 64, t.chunk, tag, init,
                                 carry)) {
            atomicOr(&p.hdr->err, 1u);
          }
        }
        if (!last) publish(p.slot_h, sidx, tag, __float_as_uint(GR ? GB : fmaf(GA, carry, GB)));
      } else {
        carry = 0.0f;
      }
      s_carry[ms][lane] = carry;
      lds_release();
      if (lane == 0) lds_store(&s_carry_ok[ms], i);
    }
  } else {
    // ------------------------------------------------------------ data waves
    // A raw word as float32. Rows of 2-byte elements are read a dword at a
    // time (the pair of channels holding the lane's) and the lane's half is
    // moved to the high half with one byte permute: bytes 1:0 (even lanes) or
    // 3:2 (odd lanes) above two zero bytes. Otherwise the 4-byte slot holds
    // the element zero-extended.
    const unsigned perm_sel = (lane & 1) ? 0x03020c0cu : 0x01000c0cu;
    auto lds_raw = [=](int b, int q, int row) -> uint32_t {
      if constexpr (ROWB == 128) {
        return *reinterpret_cast<const uint32_t*>(&s_raw[b][q][row][(lane & ~1) * 2]);
      } else {
        return *reinterpret_cast<const uint32_t*>(&s_raw[b][q][row][lane * 4]);
      }
    };
    // fused: the lane's dword of gate row wave*TS + k, through the swizzle of
    // the projection's writes (chunk c of row r at c ^ ((r >> 1) & 15));
    // row r >> 1 is wave*TS/2 + k/2, so a wave needs TS/2 lane offsets
    uint32_t gsw[FUSED ? TS / 2 : 1];
#pragma unroll
    for (int m = 0; m < (FUSED ? TS / 2 : 1); ++m) {
      gsw[m] = static_cast<uint32_t>(((lane & ~1) * 2) ^ ((((wave * TS) / 2 + m) & 15) << 3));
    }
    auto lds_gate = [=](int b, int q, int k) -> uint32_t {
      if constexpr (FUSED) {
        return *reinterpret_cast<const uint32_t*>(&s_raw[b][q][wave * TS + k][0] + gsw[k >> 1]);
      } else {
        return lds_raw(b, q, wave * TS + k);
      }
    };
    auto to_f32 = [=](uint32_t r) {
      if constexpr (ROWB == 128) return __uint_as_float(__builtin_amdgcn_perm(0u, r, perm_sel));
      else return BF ? __uint_as_float(r << 16) : __uint_as_float(r);
    };
    auto wave_steps = [=](const Tile& t) {
      const long long rem = p.L - (t.t0 + wave * TS);
      return rem <= 0 ? 0 : (rem >= TS ? TS : static_cast<int>(rem));
    };
    // h rows staged in LDS by one iteration and stored 16 bytes per lane at
    // the start of the next (two instructions a wave), so the read-back's LDS
    // latency is not waited for. Lane l stores row l / HSEG of each group of
    // 64 / HSEG rows, 16 bytes at segment l % HSEG of it.
    constexpr int HSEG = 64 * ES / 16;
    constexpr int HRPI = 64 / HSEG;
    struct Pending {
      elem* hb;   // h at the wave's first row of the staged tile
      int rn;     // rows to store
      bool on;
    };
    auto flush = [=](Pending& pd) {
      if (!pd.on) return;
      // the rows were written as elements and are read as 16-byte vectors of
      // other lanes' elements: the fence keeps the compiler from moving the
      // reads above the writes (LDS executes a wave's operations in order)
      lds_acquire();
      const int hr = lane / HSEG;
      const int hs = lane % HSEG;
#pragma unroll
      for (int g = 0; g < TS / HRPI; ++g) {
        const int row = g * HRPI + hr;
        if (row < pd.rn) {
          // wave-uniform base (the group's first row), the lane's row and
          // segment as a 32-bit element offset
          const u32x4 v = *reinterpret_cast<const u32x4*>(&s_hst[wave][row * 64 + hs * (16 / ES)]);
          Io<IO, 16 / ES>::store_nt32(pd.hb + static_cast<long long>(g * HRPI) * p.W,
                                      static_cast<unsigned>(hr) * static_cast<unsigned>(p.W) +
                                          static_cast<unsigned>(hs * (16 / ES)),
                                      v);
        }
      }
      pd.on = false;
    };
    // Waves w and w + 4 share a SIMD, whose issue arbiter prefers the older
    // wave: left alone, wave w runs ahead and wave w + 4 trails it, and the
    // tile's maps (and with them the buffers and the carry) wait for the
    // trailing wave. A wave that is ahead of its partner drops to the lower
    // priority.
    auto pace = [=](int i, int other) {
      if constexpr (NW == 8) {
        if (lane == 0) lds_store(&s_prog[wave], i);
        if (other < i) {
          __builtin_amdgcn_s_setprio(0);
        } else {
          __builtin_amdgcn_s_setprio(1);
        }
      }
    };
    // One iteration: the gates of t_i into (cal, cu, crm), and the replay of
    // t_{i-2} from (ral, ru, rrm). Returns false once t_{i-1} is past the last
    // tile (the next iteration would have nothing to replay).
    auto iteration = [=](int i, float (&cal)[TS], float (&cu)[TS], unsigned& crm, const float (&ral)[TS],
                         const float (&ru)[TS], unsigned rrm, Pending& pend) -> bool {
      const int cb = i & 1;
      const int ms = i % 3;
      const int rs_slot = (i + 1) % 3;     // slot of iteration i - 2
      // One LDS round trip for the flags the iteration checks and the data
      // they guard (tickets, the replay's carry and prefix map, the tile's
      // decay constants and reset flags): the data is read right behind its
      // flag, and read again only if the flag was not yet set (then waited
      // for). LDS runs a wave's operations in order, so data read after a
      // flag that was set is the data the flag published.
      const int f_tk = __builtin_amdgcn_readfirstlane(lds_load(&s_tk_valid));
      const int f_abort = __builtin_amdgcn_readfirstlane(lds_load(&s_abort));
      const int f_full = __builtin_amdgcn_readfirstlane(lds_load(&s_full[cb]));
      const int f_carry = __builtin_amdgcn_readfirstlane(lds_load(&s_carry_ok[rs_slot]));
      const int f_other = NW == 8 ? __builtin_amdgcn_readfirstlane(lds_load(&s_prog[wave ^ 4])) : i;
      lds_acquire();
      unsigned q_c = s_tk[i % RING];
      unsigned q_p = s_tk[(i + RING - 1) % RING];
      unsigned q_r = s_tk[(i + RING - 2) % RING];
      float c0 = s_carry[rs_slot][lane];
      float PA = s_PA[rs_slot][wave][lane];
      float PB = s_PB[rs_slot][wave][lane];
      unsigned PRm = s_PRm[rs_slot];
      unsigned rfl = s_rflag[cb][wave * TS + (lane < TS ? lane : 0)];
      uint32_t sgw = PACKED ? s_seg[cb][wave * TS + (lane < TS ? lane : 0)] : 0u;
      float k2 = s_k2[cb][lane];
      pace(i, f_other);
      flush(pend);
      if (f_tk < i) {
        lds_wait<false>(&s_tk_valid, i, &s_abort, p.hdr);
        if (lds_load(&s_abort) != 0) return false;
        q_c = s_tk[i % RING];
        q_p = s_tk[(i + RING - 1) % RING];
        q_r = s_tk[(i + RING - 2) % RING];
      } else if (f_abort != 0) {
        return false;
      }
      const Tile tc = tile_of(__builtin_amdgcn_readfirstlane(q_c));
      const Tile tp = tile_of(i > 0 ? __builtin_amdgcn_readfirstlane(q_p) : p.n_tiles);
      const Tile tr = tile_of(i > 1 ? __builtin_amdgcn_readfirstlane(q_r) : p.n_tiles);
      // the replay's incoming state (ready since the previous iteration in
      // steady state)
      float hc = 0.0f;
      int rn = 0;
      if (tr.valid) {
        if (f_carry != i - 2) {
          lds_wait<true>(&s_carry_ok[rs_slot], i - 2, &s_abort, p.hdr);
          c0 = s_carry[rs_slot][lane];
          PA = s_PA[rs_slot][wave][lane];
          PB = s_PB[rs_slot][wave][lane];
          PRm = s_PRm[rs_slot];
        }
        const bool PR = ((PRm >> wave) & 1u) != 0u;
        hc = PR ? PB : fmaf(PA, c0, PB);
        rn = wave_steps(tr);
      }
      float ck[TS / kCkpt];
      // the state after each replayed step goes to the wave's LDS rows as it
      // is computed (one element per lane and step); 8-step scheduling groups
      // bound the registers the interleaved chains keep live
      auto put_h = [=](int k, float v) {
        float h1[1] = {v};
        reinterpret_cast<typename io::R*>(&s_hst[wave][0])[k * 64 + lane] = io::pack(h1);
      };
      auto replay_step = [&](int k, bool FULL) {
        if (k % kCkpt == 0) ck[k / kCkpt] = hc;
        if (FULL) {
          hc = fmaf(ral[k], hc, ru[k]);
        } else {
          const bool rs = ((rrm >> k) & 1u) != 0u;
          const float nx = rs ? ru[k] : fmaf(ral[k], hc, ru[k]);
          hc = k < rn ? nx : hc;   // steps past L leave the state as it is
          if (PACKED && ((rrm >> (16 + k)) & 1u) != 0u && tr.active) {
            // a packed segment's last token: its final state
            p.h_last_s[static_cast<long long>(s_endseg[rs_slot][wave][k]) * W + tr.ch] = hc;
          }
        }
        put_h(k, hc);
      };
      if (tc.valid) {
        if (f_full != i) {
          lds_wait<true>(&s_full[cb], i, &s_abort, p.hdr);
          rfl = s_rflag[cb][wave * TS + (lane < TS ? lane : 0)];
          if constexpr (PACKED) sgw = s_seg[cb][wave * TS + (lane < TS ? lane : 0)];
          k2 = s_k2[cb][lane];
        }
        const int nvalid = wave_steps(tc);
        // reset flags of the wave's steps: lane k reads step k, one ballot;
        // likewise the starts and ends of packed segments
        unsigned rmask = 0, smask = 0, emask = 0;
        if (p.reset != nullptr) {
          const bool f = lane < nvalid && rfl != 0u;
          rmask = static_cast<unsigned>(__ballot(f));
        }
        if constexpr (PACKED) {
          smask = static_cast<unsigned>(__ballot(lane < nvalid && (sgw & kSegStart) != 0u));
          emask = static_cast<unsigned>(__ballot(lane < nvalid && (sgw & kSegEnd) != 0u));
          // the segments ending here, for the replay two iterations on
          if (lane < TS && ((emask >> lane) & 1u) != 0u) s_endseg[ms][wave][lane] = sgw & kSegId;
        }
        // steps that take no carry in: reset tokens and segment starts
        const unsigned cutm = rmask | smask;
        float A = 1.0f, Bv = 0.0f;
        // one step of the gates: (alpha, write) and the wave's map extended by
        // it. FULL: every step in range and no reset token, so no selects.
        auto gate_step = [&](int k, bool FULL) {
          const float xv = to_f32(lds_raw(cb, 0, wave * TS + k));
          const float ig = sigmoid_f(to_f32(lds_gate(cb, 1, k)));
          const float r = sigmoid_f(to_f32(lds_gate(cb, 2, k)));
          const float y = k2 * r;
          const float a = __builtin_amdgcn_exp2f(y);
          const float m = __builtin_amdgcn_sqrtf(one_minus_exp2(y, a) * (1.0f + a));
          if (FULL) {
            cal[k] = a;
            cu[k] = m * ig * xv;
            Bv = fmaf(a, Bv, cu[k]);
            A *= a;
          } else {
            const bool rs = ((rmask >> k) & 1u) != 0u;
            const bool cut = ((cutm >> k) & 1u) != 0u;
            float u = (rs ? 1.0f : m) * ig * xv;
            if (PACKED && ((smask >> k) & 1u) != 0u && !rs && p.h0s != nullptr) {
              // a segment's first token: its initial state decays in
              const uint32_t sg = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(sgw), k)) & kSegId;
              const float h0v = tc.active ? p.h0s[static_cast<long long>(sg) * W + tc.ch] : 0.0f;
              u = fmaf(a, h0v, u);
            }
            cal[k] = cut ? 0.0f : a;
            cu[k] = u;
            if (k < nvalid) {
              Bv = cut ? cu[k] : fmaf(cal[k], Bv, cu[k]);
              A *= cal[k];
            }
          }
        };
        if (cutm == 0u && nvalid == TS && rrm == 0u && rn == TS) {
          // common case: both tiles whole and free of reset tokens, one
          // straight-line block the scheduler can interleave
#pragma unroll
          for (int k = 0; k < TS; ++k) {
            gate_step(k, true);
            replay_step(k, true);
            if (k % 8 == 7) __builtin_amdgcn_sched_barrier(0);
          }
        } else {
          if (cutm == 0u && nvalid == TS) {
#pragma unroll
            for (int k = 0; k < TS; ++k) {
              gate_step(k, true);
              if (k % 8 == 7) __builtin_amdgcn_sched_barrier(0);
            }
          } else {
#pragma unroll
            for (int k = 0; k < TS; ++k) {
              gate_step(k, false);
              if (k % 8 == 7) __builtin_amdgcn_sched_barrier(0);
            }
          }
#pragma unroll
          for (int k = 0; k < TS; ++k) replay_step(k, false);
        }
        if constexpr (FUSED) {
          // the logits, when asked for, leave from the wave's own gate rows
          // before the buffer is released: lane l takes row wave*TS + l/8,
          // channels 8*(l%8) .. +7 (chunks 2m and 2m + 1, which the rows'
          // swizzle keeps in one aligned pair, swapped when it is odd)
          const int rr = lane >> 3, m = lane & 7;
          const int row = wave * TS + rr;
          const int f = (row >> 1) & 15;
#pragma unroll
          for (int g = 0; g < 2; ++g) {
            uint16_t* go = g ? p.gout[1] : p.gout[0];
            if (go == nullptr) continue;
            u32x4 v = *reinterpret_cast<const u32x4*>(&s_raw[cb][1 + g][row][((2 * m) ^ (f & 14)) * 8]);
            if (f & 1) v = u32x4{v[2], v[3], v[0], v[1]};
            if (rr < nvalid) *reinterpret_cast<u32x4*>(go + (tc.rowbase + tc.t0 + row) * W + tc.strip * 64 + m * 8) = v;
          }
        }
        crm = cutm | (emask << 16);
        s_A[ms][wave][lane] = A;
        s_B[ms][wave][lane] = Bv;
        if (lane == 0) s_R[ms][wave] = cutm != 0u ? 1u : 0u;
        lds_release();
        if (lane == 0) {
          lds_add(&s_maps_in[ms], 1);
          lds_add(&s_cons[cb], 1);
        }
      } else {
        // past the last tile: the ring slot is still defined (its previous
        // contents are dead, and leaving them undefined on some paths would
        // keep them alive and cost whole-array register copies)
#pragma unroll
        for (int k = 0; k < TS; ++k) {
          cal[k] = 0.0f;
          cu[k] = 0.0f;
        }
        crm = 0u;
#pragma unroll
        for (int k = 0; k < TS; ++k) replay_step(k, false);
      }
      if (tr.valid && tr.active) {
        // stores of t_{i-2}: checkpoints, h, and the final state
        const long long s0 = tr.t0 + wave * TS;
        if (p.ckpt != nullptr) {
#pragma unroll
          for (int q = 0; q < TS / kCkpt; ++q) {
            if (q * kCkpt < rn) p.ckpt[(static_cast<long long>(tr.b) * p.n_ckpt + s0 / kCkpt + q) * W + tr.ch] = ck[q];
          }
        }
        elem* hb = static_cast<elem*>(p.h) + (tr.rowbase + s0) * W + static_cast<long long>(tr.strip) * 64;
        if (p.h_wide && (tr.strip + 1) * 64 <= p.W) {
          // full strips with 16-byte aligned rows: out 16 bytes per lane at
          // the start of the next iteration
          pend.hb = hb;
          pend.rn = rn;
          pend.on = true;
        } else {
          // otherwise each lane stores its own elements, read back from LDS
          lds_acquire();
#pragma unroll
          for (int k = 0; k < TS; ++k) {
            if (k < rn) {
              const typename io::R v = reinterpret_cast<const typename io::R*>(&s_hst[wave][0])[k * 64 + lane];
              io::store_nt32(hb + static_cast<long long>(k) * W, static_cast<unsigned>(lane), v);
            }
          }
        }
        if (p.h_last != nullptr && rn > 0 && s0 + rn == p.L) p.h_last[tr.b * W + tr.ch] = hc;
      }
      return tc.valid || tp.valid;
    };
    // register ring of three tiles: iteration i writes slot i % 3 and replays
    // slot (i - 2) % 3
    float al0[TS], u0[TS], al1[TS], u1[TS], al2[TS], u2[TS];
    unsigned rm0 = 0u, rm1 = 0u, rm2 = 0u;
#pragma unroll
    for (int k = 0; k < TS; ++k) {
      al1[k] = u1[k] = al2[k] = u2[k] = 0.0f;
    }
    Pending pend{nullptr, 0, false};
    for (int i = 0;; i += 3) {
      if (!iteration(i, al0, u0, rm0, al1, u1, rm1, pend)) break;
      if (!iteration(i + 1, al1, u1, rm1, al2, u2, rm2, pend)) break;
      if (!iteration(i + 2, al2, u2, rm2, al0, u0, rm0, pend)) break;
    }
    flush(pend);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    // every workgroup has drawn its last ticket before it counts itself done;
    // the last one to finish re-arms the tickets and advances the call tag
    const unsigned prev = atomicAdd(&p.hdr->done, 1u);
    if (prev == gridDim.x - 1) {
      atomicExch(&p.hdr->done, 0u);
      advance_call(p.hdr);
    }
  }
}

// Short sequences (L <= kSerialMaxL, e.g. a decode step: L = 1 with h0 in
// and h_last out): one thread per (batch row, V channels) runs the steps in
// order. All of a thread's loads go out in one round trip and there is no
// look-back, barrier or map composition, so the call costs about a launch
// and one memory round trip. Same arithmetic as the tiled kernel; for these
// lengths the tiled kernel also runs the steps as one serial fma chain from
// h0, so the results are bitwise the same.
constexpr int kSerialMaxL = 8;
template <typename IO, int V>
__global__ __launch_bounds__(256) void fwd_serial_kernel(FwdArgs p) {
  using io = Io<IO, V>;
  using R_t = typename io::R;
  const long long groups = p.W / V;
  const long long idx = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= static_cast<long long>(p.B) * groups) return;
  const int b = static_cast<int>(idx / groups);
  const long long W = p.W;
  const long long ch = (idx - static_cast<long long>(b) * groups) * V;
  const long long rowbase = static_cast<long long>(b) * p.L;
  R_t rx[kSerialMaxL], rgx[kSerialMaxL], rga[kSerialMaxL];
  bool rs[kSerialMaxL];
  uint32_t sgw[kSerialMaxL];
#pragma unroll
  for (int k = 0; k < kSerialMaxL; ++k) {
    rx[k] = R_t{};
    rgx[k] = R_t{};
    rga[k] = R_t{};
    rs[k] = false;
    sgw[k] = 0u;
    if (k < p.L) {
      const long long off = (rowbase + k) * W + ch;
      rx[k] = io::load_nt(p.x, off);
      rgx[k] = io::load_nt(p.gx, off);
      rga[k] = io::load_nt(p.ga, off);
      rs[k] = p.reset != nullptr && p.reset[rowbase + k] != 0;
      if (p.seg != nullptr) sgw[k] = p.seg[rowbase + k];
    }
  }
  float k2[V], h[V];
#pragma unroll
  for (int j = 0; j < V; ++j) {
    float cs;
    channel_consts(p.lam[ch + j], p.c, cs, k2[j]);
    h[j] = p.h0 != nullptr ? p.h0[static_cast<long long>(b) * W + ch + j] : 0.0f;
  }
#pragma unroll
  for (int k = 0; k < kSerialMaxL; ++k) {
    if (k < p.L) {
      if (p.ckpt != nullptr && k % kCkpt == 0) {
        store_f32v<V>(p.ckpt + (static_cast<long long>(b) * p.n_ckpt + k / kCkpt) * W + ch, h);
      }
      float xv[V], gxv[V], gav[V];
      io::unpack(rx[k], xv);
      io::unpack(rgx[k], gxv);
      io::unpack(rga[k], gav);
      // a packed segment's first token starts from the segment's initial
      // state (zero without h0s)
      const bool start = (sgw[k] & kSegStart) != 0u;
      const long long sg = static_cast<long long>(sgw[k] & kSegId);
#pragma unroll
      for (int j = 0; j < V; ++j) {
        const float ig = sigmoid_f(gxv[j]);
        const float r = sigmoid_f(gav[j]);
        const float y = k2[j] * r;
        const float a = __builtin_amdgcn_exp2f(y);
        const float m = __builtin_amdgcn_sqrtf(one_minus_exp2(y, a) * (1.0f + a));
        const float hp = start ? (p.h0s != nullptr ? p.h0s[sg * W + ch + j] : 0.0f) : h[j];
        h[j] = rs[k] ? ig * xv[j] : fmaf(a, hp, m * ig * xv[j]);
      }
      io::store_nt(p.h, (rowbase + k) * W + ch, io::pack(h));
      if ((sgw[k] & kSegEnd) != 0u && p.h_last_s != nullptr) store_f32v<V>(p.h_last_s + sg * W + ch, h);
    }
  }
  if (p.h_last != nullptr) store_f32v<V>(p.h_last + static_cast<long long>(b) * W + ch, h);
}

// ------------------------------------------------------------------ backward
//
// The reverse recurrence g_t = dh_t + alpha_{t+1} g_{t+1} runs as a single
// persistent pass over tiles in reverse chunk order, the mirror image of the
// forward: a tile is one batch row, a strip of 64 channels (one per lane) and
// T = NW * 8 steps, wave w owning steps 8w .. 8w+7 (one checkpoint interval,
// whose entering state the forward stored). The carry a tile needs enters its
// last step from the later chunks, so the look-back runs over later chunks.
// A workgroup has NW data waves, two control waves and two load waves, joined
// by one-directional LDS flags. With t_i the workgroup's i-th tile:
//   load wave i%2 : once the data waves are done with the buffers t_i goes
//                   to, streams its raw gate_a and dh words into buffer i%2,
//                   its x and gate_x words and checkpoint rows into buffer
//                   i%4, and the reset flags, with global_load_lds, and
//                   evaluates the decay constants;
//   data waves    : in iteration i, turn gate_a and dh of their steps of t_i
//                   into the decays a and keep (a, r, dh) per step (a register
//                   ring of three tiles), reduce their steps to the reverse
//                   map G -> R ? B : A*G + B and report it; then wait for the
//                   carry of t_{i-2}, recompute the forward through their
//                   steps of it from the checkpoint and run its reverse pass,
//                   writing dx, dgate_x and dgate_a; the last wave to finish
//                   sums the waves' lambda-gradient parts in wave order into
//                   the tile's partial;
//   control wave i%2 : one look-back round ahead of the maps; once every data
//                   wave has reported t_i, writes the suffix maps each wave's
//                   reverse pass starts from, publishes the tile's map, runs
//                   the look-back and publishes the outgoing carry.
// The carry of t_i is needed two iterations after its maps are in, which
// hides the look-back's latency behind the work of a whole iteration.
// Per step, with G the carry arriving from the next step:
//   g = G + dh;  dx = g*cx;  dgate_x = g*cgx;  dgate_a = g*cga;
//   lambda partial += g*cl;  G <- alpha*g  (0 through a reset token)
// where cx = mult*i, cgx = mult*i*x*(1-i), dl = g*a*(h_prev - a*i*x/m) off
// reset tokens (0 on them), cl = dl/g * r, cga = cl * c_s * (1 - r). The
// per-tile partials are summed per channel in a fixed order by
// bwd_dlam_kernel, so the backward is deterministic run to run.

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
  // packed sequences (batch row 0 only; nullptr otherwise): per-token
  // segment word, the segments' initial states and the gradients on their
  // final states in, the gradients on their initial states out [n_segments, W]
  const uint32_t* seg;
  const float* h0s;
  const float* dh_last_s;
  float* dh0s;
  Header* hdr;
  u64* slot_a;           // published reverse map A (a reset in the sign bit)
  u64* slot_b;           // published reverse map B
  u64* slot_h;           // published carry leaving the tile's first step
  float* part;           // lambda-gradient partial per tile and channel
  long long L;
  long long n_ckpt;
  int B;
  int W;
  int n_strips;
  int n_chunks;
  unsigned n_tiles;
  float c;
  bool out_wide;         // output rows start 16-byte aligned
};

template <typename IO, int NW, bool WIDE, bool PACKED>
__global__ __launch_bounds__((NW + 4) * 64) void bwd_kernel(BwdArgs p) {
  using elem = typename IO::elem;
  using io = Io<IO, 1>;
  constexpr bool BF = std::is_same<IO, BF16>::value;
  constexpr int ES = static_cast<int>(sizeof(elem));
  constexpr int TS = kCkpt;
  constexpr int T = NW * TS;
  constexpr int ROWB = WIDE ? 64 * ES : 256;
  constexpr int SEG = ROWB / 16;
  constexpr int RPI = 64 / SEG;
  constexpr int K = RGLRU_FWD_LOOKBACK;
  constexpr int RING = 16;
  constexpr int NFL = T < 64 ? 64 : T;
  constexpr int CTRL0 = NW, LOAD0 = NW + 2;
  constexpr bool STAGE = BF;               // bf16 outputs go out 16 bytes per lane through LDS
  static_assert(!WIDE || T % RPI == 0, "a tile is a whole number of 16-byte-per-lane instructions");
  static_assert(NFL % 64 == 0 && NFL <= 128, "reset flags: at most two instructions");
  static_assert(NW <= 32, "reset flags of the waves fit one mask word");

  // raw words: gate_a and dh feed a tile's maps (buffer i % 2), x and gate_x
  // its reverse pass two iterations later (buffer i % 4, with the checkpoint
  // rows and the decay constants)
  __shared__ __attribute__((aligned(16))) unsigned char s_rm[2][2][T][ROWB];
  __shared__ __attribute__((aligned(16))) unsigned char s_rx[4][2][T][ROWB];
  __shared__ __attribute__((aligned(16))) float s_ck[4][NW][64];   // state entering each wave's first step
  __shared__ unsigned s_rflag[2][NFL];
  __shared__ uint32_t s_seg[2][NFL];  // segment words (packed sequences)
  __shared__ uint32_t s_sseg[3][NW][TS];     // a wave's segment starts, per ring slot
  __shared__ float s_k2[4][64];
  __shared__ float s_cs[4][64];
  // a wave's reverse map; the control wave overwrites it with the composite
  // of the maps of the waves after that wave (what the wave's reverse pass
  // starts from)
  __shared__ float s_A[3][NW][64];
  __shared__ float s_B[3][NW][64];
  __shared__ unsigned s_R[3][NW];
  __shared__ unsigned s_SRm[3];       // bit w: a reset inside the waves after wave w
  __shared__ float s_carry[3][64];
  __shared__ float s_dl[3][NW][64];   // each wave's part of a tile's lambda gradient
  __shared__ __attribute__((aligned(16))) elem s_ost[STAGE ? NW : 1][3][TS * 64];
  __shared__ unsigned s_tk[RING];
  __shared__ unsigned s_tag;
  __shared__ int s_tk_valid;
  __shared__ int s_full[2];
  __shared__ int s_cons_m[2];         // data-wave maps done on gate_a/dh buffer b
  __shared__ int s_cons_x[4];         // data-wave reverse passes done on x/gate_x buffer b
  __shared__ int s_maps_in[3];
  __shared__ int s_dl_in[3];
  __shared__ int s_dl_done[3];        // tile (iteration) whose parts slot s last summed
  __shared__ int s_carry_ok[3];       // iteration whose incoming carry slot s holds
  __shared__ int s_prog[NW];          // iteration each data wave is in
  __shared__ int s_abort;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const unsigned rows = static_cast<unsigned>(p.B) * static_cast<unsigned>(p.n_strips);
  const long long W = p.W;

  if (threadIdx.x == 0) {
    s_tk_valid = -1;
    s_full[0] = s_full[1] = -1;
    s_cons_m[0] = s_cons_m[1] = 0;
    s_cons_x[0] = s_cons_x[1] = s_cons_x[2] = s_cons_x[3] = 0;
#pragma unroll
    for (int s = 0; s < 3; ++s) {
      s_maps_in[s] = 0;
      s_dl_in[s] = 0;
      s_dl_done[s] = s - 3;
      s_carry_ok[s] = -1;
    }
#pragma unroll
    for (int w = 0; w < NW; ++w) s_prog[w] = -1;
    s_abort = 0;
  }
  __syncthreads();

  struct Tile {
    bool valid, active;
    int chunk, b, strip, ch;
    unsigned id;                // chunk-major index (slot and partial addressing)
    long long t0, rowbase;
  };
  // ticket q -> chunk n_chunks - 1 - q / rows (latest chunk first)
  auto tile_of = [=](unsigned q) {
    Tile t;
    t.valid = q < p.n_tiles;
    const unsigned qq = t.valid ? q : 0u;
    const unsigned cq = qq / rows;
    const int row = static_cast<int>(qq - cq * rows);
    t.chunk = p.n_chunks - 1 - static_cast<int>(cq);
    t.id = static_cast<unsigned>(t.chunk) * rows + static_cast<unsigned>(row);
    t.b = row / p.n_strips;
    t.strip = row - t.b * p.n_strips;
    t.ch = t.strip * 64 + lane;
    t.active = t.ch < p.W;
    t.t0 = static_cast<long long>(t.chunk) * T;
    t.rowbase = static_cast<long long>(t.b) * p.L;
    return t;
  };
  auto ticket_tile = [=](u64 v, unsigned k) {
    const unsigned q = static_cast<unsigned>(v) + k;
    return q < p.n_tiles ? q : p.n_tiles;
  };
  auto wave_steps = [=](const Tile& t, int w) {
    const long long rem = p.L - (t.t0 + w * TS);
    return rem <= 0 ? 0 : (rem >= TS ? TS : static_cast<int>(rem));
  };

  if (wave >= LOAD0) {
    // ------------------------------------------------------------ load waves
    __builtin_amdgcn_s_setprio(3);
    const int j = wave - LOAD0;
    if (j == 0) {
      u64 v = 0;
      if (lane == 0) v = atomicAdd(&p.hdr->counter, 2ull);
      v = uniform_u64(v);
      if (lane == 0) {
        s_tk[0] = ticket_tile(v, 0);
        s_tk[1] = ticket_tile(v, 1);
        s_tag = static_cast<unsigned>(v >> 32) + 1u;
      }
      lds_release();
      if (lane == 0) lds_store(&s_tk_valid, 1);
    }
    const unsigned char* src[4] = {
        static_cast<const unsigned char*>(p.ga), static_cast<const unsigned char*>(p.dh),
        static_cast<const unsigned char*>(p.x), static_cast<const unsigned char*>(p.gx)};
    const long long row_bytes = W * ES;
    for (int i = j;; i += 2) {
      const int xb = i & 3;
      lds_wait<false, kHelperSleep>(&s_tk_valid, i, &s_abort, p.hdr);
      const Tile t = tile_of(__builtin_amdgcn_readfirstlane(s_tk[i % RING]));
      // the maps of t_{i-2} and the reverse pass of t_{i-4} are done with
      // the buffers t_i goes to
      lds_wait<false, kHelperSleep>(&s_cons_m[j], NW * (i / 2), &s_abort, p.hdr);
      lds_wait<false, kHelperSleep>(&s_cons_x[xb], NW * (i / 4), &s_abort, p.hdr);
      if (lds_load(&s_abort) != 0) break;
      if (!t.valid) {
        if (lane == 0) lds_store(&s_full[j], i);
        break;
      }
      auto dst_of = [&](int q, int row) -> unsigned char* {
        return q < 2 ? &s_rm[j][q][row][0] : &s_rx[xb][q - 2][row][0];
      };
      float lam = 0.0f;
      if (t.active) lam = p.lam[t.ch];
      const long long strip_b = static_cast<long long>(t.strip) * 64 * ES;
      const long long tile_off = (t.rowbase + t.t0) * row_bytes + strip_b;
      const long long lim = p.L - 1 - t.t0;
      if constexpr (WIDE) {
        const int r = lane / SEG;
        const unsigned seg = static_cast<unsigned>(lane % SEG) * 16u;
        const unsigned col = strip_b + seg < row_bytes ? seg : 0u;
        if (t.t0 + T <= p.L) {
          const unsigned step = static_cast<unsigned>(RPI) * static_cast<unsigned>(row_bytes);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            gbyte* base = uniform_gptr(src[q] + tile_off);
            unsigned off = static_cast<unsigned>(r) * static_cast<unsigned>(row_bytes) + col;
            unsigned char* dst = dst_of(q, 0);
#pragma unroll 4
            for (int g = 0; g < T / RPI; ++g) {
              lds_dma16(base + off, dst);
              off += step;
              dst += 1024;
            }
          }
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            gbyte* base = uniform_gptr(src[q] + tile_off);
            for (int g = 0; g < T / RPI; ++g) {
              const long long row = g * RPI + r;
              const long long off = (row < lim ? row : lim) * row_bytes + col;
              lds_dma16(base + off, dst_of(q, g * RPI));
            }
          }
        }
      } else {
        const unsigned col = t.active ? static_cast<unsigned>(lane * ES) : 0u;
#pragma unroll 2
        for (int k = 0; k < T; ++k) {
          const long long row = k < lim ? k : lim;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            gbyte* base = uniform_gptr(src[q] + tile_off + row * row_bytes);
            __builtin_amdgcn_global_load_lds(const_cast<gbyte_w*>(base + col), dst_of(q, k), ES, 0, 0);
          }
        }
      }
      // checkpoint rows (float32, one per wave; waves past L re-read row 0 of
      // the tile, never used) and reset flags
      {
        const unsigned col = t.active ? static_cast<unsigned>(lane * 4) : 0u;
        const long long ck0 = static_cast<long long>(t.b) * p.n_ckpt + t.t0 / TS;
        for (int w = 0; w < NW; ++w) {
          const long long kr = t.t0 + w * TS < p.L ? w : 0;
          gbyte* base = uniform_gptr(p.ckpt + (ck0 + kr) * W + static_cast<long long>(t.strip) * 64);
          __builtin_amdgcn_global_load_lds(const_cast<gbyte_w*>(base + col), &s_ck[xb][w][0], 4, 0, 0);
        }
      }
      if (p.reset != nullptr) {
#pragma unroll
        for (int h = 0; h < NFL / 64; ++h) {
          const long long st = h * 64 + lane;
          const long long tk = t.t0 + (st < lim ? st : lim);
          __builtin_amdgcn_global_load_lds(p.reset + t.rowbase + tk, &s_rflag[j][h * 64], 1, 0, 0);
        }
      }
      if constexpr (PACKED) {
#pragma unroll
        for (int h = 0; h < NFL / 64; ++h) {
          const long long st = h * 64 + lane;
          const long long tk = t.t0 + (st < lim ? st : lim);
          __builtin_amdgcn_global_load_lds(const_cast<uint32_t*>(p.seg) + t.rowbase + tk, &s_seg[j][h * 64], 4, 0, 0);
        }
      }
      u64 nxt = 0;
      if (j == 0 && lane == 0) nxt = atomicAdd(&p.hdr->counter, 2ull);
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      {
        float cs = 0.0f, k2 = 0.0f;
        if (t.active) channel_consts(lam, p.c, cs, k2);
        s_k2[xb][lane] = k2;
        s_cs[xb][lane] = cs;
      }
      if (j == 0) {
        nxt = uniform_u64(nxt);
        if (lane == 0) {
          s_tk[(i + 2) % RING] = ticket_tile(nxt, 0);
          s_tk[(i + 3) % RING] = ticket_tile(nxt, 1);
        }
      }
      lds_release();
      if (lane == 0) {
        if (j == 0) lds_store(&s_tk_valid, i + 3);
        lds_store(&s_full[j], i);
      }
    }
  } else if (wave >= CTRL0) {
    // ------------------------------------------------------------ control waves
    // Control wave c handles the tiles of iterations c, c + 2, ...: one
    // speculative look-back round; once every data wave has reported t_i,
    // the suffix maps each wave's reverse pass starts from; publishes the
    // tile's map (the latest chunk publishes its outgoing carry instead), runs
    // the look-back and publishes the outgoing carry.
    __builtin_amdgcn_s_setprio(3);
    const int c = wave - CTRL0;
    unsigned tag = 0;
    for (int i = c;; i += 2) {
      lds_wait<false, kHelperSleep>(&s_tk_valid, i, &s_abort, p.hdr);
      if (lds_load(&s_abort) != 0) break;
      if (i == c) tag = __builtin_amdgcn_readfirstlane(s_tag);
      const Tile tc = tile_of(__builtin_amdgcn_readfirstlane(s_tk[i % RING]));
      if (!tc.valid) break;
      const int ms = i % 3;
      const size_t sidx = static_cast<size_t>(tc.id) * 64 + lane;
      const bool latest = tc.chunk == p.n_chunks - 1;
      const float init = (tc.active && p.dh_last != nullptr) ? p.dh_last[tc.b * W + tc.ch] : 0.0f;
      // one look-back round before this tile's maps are in (it needs only the
      // later chunks' words)
      float carry = init;
      bool found = true;
      if (tc.active && !latest) {
        found = look_back_round<K, true>(p.slot_a, p.slot_b, p.slot_h, static_cast<long long>(tc.id) * 64,
                                   static_cast<unsigned>(lane), -static_cast<long long>(rows) * 64,
                                   p.n_chunks - 1 - tc.chunk, tag, init, carry);
      }
      // reports count per ring slot: a data wave may report t_{i+1} or t_{i+2}
      // before another reports t_i
      lds_wait<false, kHelperSleep>(&s_maps_in[ms], NW * (i / 3 + 1), &s_abort, p.hdr);
      if (lds_load(&s_abort) != 0) break;
      float Aw[NW], Bw[NW];
      unsigned Rw[NW];
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        Rw[w] = s_R[ms][w];
        Aw[w] = s_A[ms][w][lane];
        Bw[w] = s_B[ms][w][lane];
      }
      float GA = 1.0f, GB = 0.0f;
      bool GR = false;
      unsigned srbits = 0u;
#pragma unroll
      for (int w = NW - 1; w >= 0; --w) {
        s_A[ms][w][lane] = GA;
        s_B[ms][w][lane] = GB;
        srbits |= GR ? (1u << w) : 0u;
        GB = Rw[w] != 0u ? Bw[w] : fmaf(Aw[w], GB, Bw[w]);
        GA *= Aw[w];
        GR = GR || Rw[w] != 0u;
      }
      if (lane == 0) s_SRm[ms] = srbits;
      if (tc.active) {
        if (!found) {
          if (tc.chunk > 0) {
            publish(p.slot_a, sidx, tag, encode_a(GA, GR));
            publish(p.slot_b, sidx, tag, __float_as_uint(GB));
          }
          if (!look_back_wave<K, true>(p.slot_a, p.slot_b, p.slot_h, static_cast<long long>(tc.id) * 64,
                                 static_cast<unsigned>(lane), -static_cast<long long>(rows) * 64,
                                 p.n_chunks - 1 - tc.chunk, tag, init, carry)) {
            atomicOr(&p.hdr->err, 1u);
          }
        }
        if (tc.chunk > 0) publish(p.slot_h, sidx, tag, __float_as_uint(GR ? GB : fmaf(GA, carry, GB)));
      } else {
        carry = 0.0f;
      }
      s_carry[ms][lane] = carry;
      lds_release();
      if (lane == 0) lds_store(&s_carry_ok[ms], i);
    }
  } else {
    // ------------------------------------------------------------ data waves
    const unsigned perm_sel = (lane & 1) ? 0x03020c0cu : 0x01000c0cu;
    auto lds_word = [=](const unsigned char (&buf)[T][ROWB], int row) -> uint32_t {
      if constexpr (ROWB == 128) {
        return *reinterpret_cast<const uint32_t*>(&buf[row][(lane & ~1) * 2]);
      } else {
        return *reinterpret_cast<const uint32_t*>(&buf[row][lane * 4]);
      }
    };
    auto to_f32 = [=](uint32_t r) {
      if constexpr (ROWB == 128) return __uint_as_float(__builtin_amdgcn_perm(0u, r, perm_sel));
      else return BF ? __uint_as_float(r << 16) : __uint_as_float(r);
    };
    // outputs staged in LDS by one iteration and stored 16 bytes per lane at
    // the start of the next (lane l: row l / HSEG, segment l % HSEG)
    constexpr int HSEG = 64 * ES / 16;
    constexpr int HRPI = 64 / HSEG;
    struct Pending {
      long long base;   // element offset of the wave's first row in the outputs
      int rn;
      bool on;
    };
    auto flush = [=](Pending& pd) {
      if constexpr (STAGE) {
        if (!pd.on) return;
        lds_acquire();
        const int hr = lane / HSEG;
        const int hs = lane % HSEG;
        void* outs[3] = {p.dx, p.dgx, p.dga};
#pragma unroll
        for (int q = 0; q < 3; ++q) {
#pragma unroll
          for (int g = 0; g < TS / HRPI; ++g) {
            const int row = g * HRPI + hr;
            if (row < pd.rn) {
              const u32x4 v = *reinterpret_cast<const u32x4*>(&s_ost[wave][q][row * 64 + hs * (16 / ES)]);
              Io<IO, 16 / ES>::store_nt32(static_cast<elem*>(outs[q]) + pd.base + static_cast<long long>(g * HRPI) * p.W,
                                          static_cast<unsigned>(hr) * static_cast<unsigned>(p.W) +
                                              static_cast<unsigned>(hs * (16 / ES)),
                                          v);
            }
          }
        }
        pd.on = false;
      }
    };
    // Waves w and w + 4 share a SIMD, whose issue arbiter prefers the older
    // wave: left alone, wave w runs ahead and wave w + 4 trails it by most of
    // an iteration, so the tile's maps (and with them the buffers and the
    // carry) wait for the trailing wave while the SIMD runs one wave at a
    // time. A wave that is ahead of its partner drops to the lower priority.
    auto pace = [=](int i, int other) {
      if constexpr (NW == 8) {
        if (lane == 0) lds_store(&s_prog[wave], i);
        if (other < i) {
          __builtin_amdgcn_s_setprio(0);
        } else {
          __builtin_amdgcn_s_setprio(1);
        }
      }
    };
    // One iteration: the maps of t_i from gate_a and dh, keeping (a, r, dh)
    // per step in the ring slot (ca, cr, cd, cm); then the reverse pass of
    // t_{i-2} from its slot (pa, pr, pd, pm), the recomputed forward through
    // its steps and its incoming carry. Returns false once t_{i-1} is past
    // the last tile (the next iteration would have nothing to reverse).
    auto iteration = [=](int i, float (&ca)[TS], float (&cr)[TS], float (&cd)[TS], unsigned& cm,
                         const float (&pa)[TS], const float (&pr)[TS], const float (&pd)[TS], unsigned pm,
                         Pending& pend) -> bool {
      const int mb = i & 1;
      const int rs3 = (i + 1) % 3;       // ring slot of t_{i-2}
      // One LDS round trip for the flags the iteration checks and the data
      // they guard (tickets, the tile's reset flags and decay constants, the
      // reverse pass's carry and suffix map): the data is read right behind
      // its flag, and read again only if the flag was not yet set (then
      // waited for). LDS runs a wave's operations in order, so data read
      // after a flag that was set is the data the flag published.
      const int f_tk = __builtin_amdgcn_readfirstlane(lds_load(&s_tk_valid));
      const int f_abort = __builtin_amdgcn_readfirstlane(lds_load(&s_abort));
      const int f_full = __builtin_amdgcn_readfirstlane(lds_load(&s_full[mb]));
      const int f_carry = __builtin_amdgcn_readfirstlane(lds_load(&s_carry_ok[rs3]));
      const int f_dl = __builtin_amdgcn_readfirstlane(lds_load(&s_dl_done[rs3]));
      const int f_other = NW == 8 ? __builtin_amdgcn_readfirstlane(lds_load(&s_prog[wave ^ 4])) : i;
      lds_acquire();
      unsigned q_c = s_tk[i % RING];
      unsigned q_p = s_tk[(i + RING - 1) % RING];
      unsigned q_r = s_tk[(i + RING - 2) % RING];
      unsigned rfl = s_rflag[mb][wave * TS + (lane < TS ? lane : 0)];
      uint32_t sgw = PACKED ? s_seg[mb][wave * TS + (lane < TS ? lane : 0)] : 0u;
      float k2m = s_k2[i & 3][lane];
      float c0 = s_carry[rs3][lane];
      float SA = s_A[rs3][wave][lane];
      float SB = s_B[rs3][wave][lane];
      unsigned SRm = s_SRm[rs3];
      pace(i, f_other);
      flush(pend);
      if (f_tk < i) {
        lds_wait<false>(&s_tk_valid, i, &s_abort, p.hdr);
        if (lds_load(&s_abort) != 0) return false;
        q_c = s_tk[i % RING];
        q_p = s_tk[(i + RING - 1) % RING];
        q_r = s_tk[(i + RING - 2) % RING];
      } else if (f_abort != 0) {
        return false;
      }
      const Tile tc = tile_of(__builtin_amdgcn_readfirstlane(q_c));
      const Tile tp = tile_of(i > 0 ? __builtin_amdgcn_readfirstlane(q_p) : p.n_tiles);
      const Tile tr = tile_of(i > 1 ? __builtin_amdgcn_readfirstlane(q_r) : p.n_tiles);
      if (tc.valid) {
        const int ms = i % 3;
        if (f_full != i) {
          lds_wait<true>(&s_full[mb], i, &s_abort, p.hdr);
          rfl = s_rflag[mb][wave * TS + (lane < TS ? lane : 0)];
          if constexpr (PACKED) sgw = s_seg[mb][wave * TS + (lane < TS ? lane : 0)];
          k2m = s_k2[i & 3][lane];
        }
        const int nvalid = wave_steps(tc, wave);
        unsigned rmask = 0, smask = 0, emask = 0;
        if (p.reset != nullptr) {
          const bool f = lane < nvalid && rfl != 0u;
          rmask = static_cast<unsigned>(__ballot(f));
        }
        if constexpr (PACKED) {
          smask = static_cast<unsigned>(__ballot(lane < nvalid && (sgw & kSegStart) != 0u));
          emask = static_cast<unsigned>(__ballot(lane < nvalid && (sgw & kSegEnd) != 0u));
          // the segments starting here, for the reverse pass two iterations on
          if (lane < TS && ((smask >> lane) & 1u) != 0u) s_sseg[ms][wave][lane] = sgw & kSegId;
        }
        // steps that pass no gradient back: reset tokens and segment starts
        const unsigned cutm = rmask | smask;
        const float k2 = k2m;
#pragma unroll
        for (int k = 0; k < TS; ++k) {
          const float r = sigmoid_f(to_f32(lds_word(s_rm[mb][0], wave * TS + k)));
          cd[k] = to_f32(lds_word(s_rm[mb][1], wave * TS + k));
          cr[k] = r;
          ca[k] = __builtin_amdgcn_exp2f(k2 * r);
        }
        lds_release();
        if (lane == 0) lds_add(&s_cons_m[mb], 1);
        if (PACKED && emask != 0u && p.dh_last_s != nullptr) {
          // a packed segment's last token also carries the gradient on the
          // segment's final state
#pragma unroll
          for (int k = 0; k < TS; ++k) {
            if (((emask >> k) & 1u) != 0u && tc.active) {
              const uint32_t sg = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(sgw), k)) & kSegId;
              cd[k] += p.dh_last_s[static_cast<long long>(sg) * W + tc.ch];
            }
          }
        }
        // the wave's reverse map G_in -> G_out, latest step first
        // (a reset token passes nothing on: a select, so not even a NaN
        // arriving from a later step crosses it)
        float A = 1.0f, Bv = 0.0f;
        if (cutm == 0u && nvalid == TS) {
#pragma unroll
          for (int k = TS - 1; k >= 0; --k) {
            Bv = ca[k] * (Bv + cd[k]);
            A = ca[k] * A;
          }
        } else {
#pragma unroll
          for (int k = TS - 1; k >= 0; --k) {
            if (k < nvalid) {
              const bool cut = ((cutm >> k) & 1u) != 0u;
              Bv = cut ? 0.0f : ca[k] * (Bv + cd[k]);
              A = cut ? 0.0f : ca[k] * A;
            }
          }
        }
        cm = rmask | (smask << 16);
        s_A[ms][wave][lane] = A;
        s_B[ms][wave][lane] = Bv;
        if (lane == 0) s_R[ms][wave] = cutm != 0u ? 1u : 0u;
        lds_release();
        if (lane == 0) lds_add(&s_maps_in[ms], 1);
      } else {
#pragma unroll
        for (int k = 0; k < TS; ++k) ca[k] = cr[k] = cd[k] = 0.0f;
        cm = 0u;
      }
      if (tr.valid) {
        // reverse pass of t_{i-2} from the carry entering its last step
        const int xb = (i - 2) & 3;
        if (f_carry != i - 2) {
          lds_wait<true>(&s_carry_ok[rs3], i - 2, &s_abort, p.hdr);
          c0 = s_carry[rs3][lane];
          SA = s_A[rs3][wave][lane];
          SB = s_B[rs3][wave][lane];
          SRm = s_SRm[rs3];
        }
        const int rn = wave_steps(tr, wave);
        const bool SR = ((SRm >> wave) & 1u) != 0u;
        float G = SR ? SB : fmaf(SA, c0, SB);
        const float k2 = s_k2[xb][lane];
        const float cs = s_cs[xb][lane];
        float h = s_ck[xb][wave][lane];
        // recompute the forward through the wave's steps, per step the
        // coefficients of the reverse pass, then the reverse pass itself.
        // FULL: every step in range and no reset token, so no selects.
        float ox[TS], ogx[TS], oga[TS];
        float dl = 0.0f;
        auto reverse = [&](auto full_tag) {
          constexpr bool FULL = decltype(full_tag)::value;
          float cx[TS], cgx[TS], cga[TS], cl[TS];
#pragma unroll
          for (int k = 0; k < TS; ++k) {
            const float xv = to_f32(lds_word(s_rx[xb][0], wave * TS + k));
            const float iv = sigmoid_f(to_f32(lds_word(s_rx[xb][1], wave * TS + k)));
            const float r = pr[k];
            const float a = pa[k];
            const bool rs = FULL ? false : ((pm >> k) & 1u) != 0u;
            // a packed segment's first token starts from the segment's
            // initial state (zero without h0s), not the carry
            float hp = h;
            if (PACKED && !FULL && ((pm >> (16 + k)) & 1u) != 0u) {
              hp = (tr.active && p.h0s != nullptr)
                       ? p.h0s[static_cast<long long>(s_sseg[rs3][wave][k]) * W + tr.ch]
                       : 0.0f;
            }
            const float y = k2 * r;
            const float w1 = one_minus_exp2(y, a) * (1.0f + a);  // 1 - a^2
            // 1 / m. Below the smallest normal float, 1 - a^2 comes from a
            // logit under about -87 (r = 0 or subnormal, a = 1): m is then
            // under 1e-19, every gradient through m vanishes in the limit, and
            // v_rsq_f32 would read a subnormal as 0 and return inf. Taking
            // 1/m as 0 there keeps inf and inf * 0 out of the gradients.
            const float rsq = w1 >= 1.17549435e-38f ? __builtin_amdgcn_rsqf(w1) : 0.0f;
            const float m = w1 * rsq;
            const float mult = rs ? 1.0f : m;
            const float ix = iv * xv;
            const float z = rs ? 0.0f : a * (hp - a * ix * rsq);
            const float uw = mult * ix;
            h = rs ? uw : fmaf(a, hp, uw);
            cx[k] = mult * iv;
            cgx[k] = uw * (1.0f - iv);
            cl[k] = z * r;
            cga[k] = cl[k] * fmaf(-cs, r, cs);
          }
          lds_release();
          if (lane == 0) lds_add(&s_cons_x[xb], 1);
#pragma unroll
          for (int k = TS - 1; k >= 0; --k) {
            const float g = G + pd[k];
            ox[k] = g * cx[k];
            ogx[k] = g * cgx[k];
            oga[k] = g * cga[k];
            if (FULL) {
              dl = fmaf(g, cl[k], dl);
              G = pa[k] * g;
            } else {
              const bool in = k < rn;
              const bool rs = ((pm >> k) & 1u) != 0u;
              const bool ss = PACKED && ((pm >> (16 + k)) & 1u) != 0u;
              dl = in ? fmaf(g, cl[k], dl) : dl;
              if (ss && in && tr.active && p.dh0s != nullptr) {
                // what would pass to the previous token goes to the
                // segment's initial state instead
                p.dh0s[static_cast<long long>(s_sseg[rs3][wave][k]) * W + tr.ch] = rs ? 0.0f : pa[k] * g;
              }
              G = in ? ((rs || ss) ? 0.0f : pa[k] * g) : G;
            }
          }
        };
        if (pm == 0u && rn == TS) {
          reverse(std::true_type{});
        } else {
          reverse(std::false_type{});
        }
        // the tile's lambda-gradient partial: the last wave to report sums
        // the waves' parts in wave order
        if (f_dl != i - 5) lds_wait<true>(&s_dl_done[rs3], i - 5, &s_abort, p.hdr);
        s_dl[rs3][wave][lane] = tr.active ? dl : 0.0f;
        lds_release();
        int prev = 0;
        if (lane == 0) prev = __hip_atomic_fetch_add(&s_dl_in[rs3], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        prev = __builtin_amdgcn_readfirstlane(prev);
        if (prev + 1 == NW * ((i - 2) / 3 + 1)) {
          lds_acquire();
          float sum = 0.0f;
#pragma unroll
          for (int w = 0; w < NW; ++w) sum += s_dl[rs3][w][lane];
          p.part[static_cast<size_t>(tr.id) * 64 + lane] = sum;
          lds_release();
          if (lane == 0) lds_store(&s_dl_done[rs3], i - 2);
        }
        if (tr.active) {
          if (tr.chunk == 0 && wave == 0 && p.dh0 != nullptr) p.dh0[tr.b * W + tr.ch] = G;
          const long long s0 = tr.t0 + wave * TS;
          const long long base = (tr.rowbase + s0) * W + static_cast<long long>(tr.strip) * 64;
          if (STAGE && p.out_wide && (tr.strip + 1) * 64 <= p.W) {
#pragma unroll
            for (int k = 0; k < TS; ++k) {
              float v0[1] = {ox[k]}, v1[1] = {ogx[k]}, v2[1] = {oga[k]};
              reinterpret_cast<typename io::R*>(&s_ost[0][0][0])[(wave * 3 + 0) * TS * 64 + k * 64 + lane] = io::pack(v0);
              reinterpret_cast<typename io::R*>(&s_ost[0][0][0])[(wave * 3 + 1) * TS * 64 + k * 64 + lane] = io::pack(v1);
              reinterpret_cast<typename io::R*>(&s_ost[0][0][0])[(wave * 3 + 2) * TS * 64 + k * 64 + lane] = io::pack(v2);
            }
            pend.base = base;
            pend.rn = rn;
            pend.on = true;
          } else {
#pragma unroll
            for (int k = 0; k < TS; ++k) {
              if (k < rn) {
                float v0[1] = {ox[k]}, v1[1] = {ogx[k]}, v2[1] = {oga[k]};
                const long long ro = base + static_cast<long long>(k) * W;
                io::store_nt32(static_cast<elem*>(p.dx) + ro, static_cast<unsigned>(lane), io::pack(v0));
                io::store_nt32(static_cast<elem*>(p.dgx) + ro, static_cast<unsigned>(lane), io::pack(v1));
                io::store_nt32(static_cast<elem*>(p.dga) + ro, static_cast<unsigned>(lane), io::pack(v2));
              }
            }
          }
        }
      }
      return tc.valid || tp.valid;
    };
    float a0[TS], r0[TS], d0[TS], a1[TS], r1[TS], d1[TS], a2[TS], r2[TS], d2[TS];
    unsigned m0 = 0u, m1 = 0u, m2 = 0u;
#pragma unroll
    for (int k = 0; k < TS; ++k) a1[k] = r1[k] = d1[k] = a2[k] = r2[k] = d2[k] = 0.0f;
    Pending pend{0, 0, false};
    for (int i = 0;; i += 3) {
      if (!iteration(i, a0, r0, d0, m0, a1, r1, d1, m1, pend)) break;
      if (!iteration(i + 1, a1, r1, d1, m1, a2, r2, d2, m2, pend)) break;
      if (!iteration(i + 2, a2, r2, d2, m2, a0, r0, d0, m0, pend)) break;
    }
    flush(pend);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev = atomicAdd(&p.hdr->done, 1u);
    if (prev == gridDim.x - 1) {
      atomicExch(&p.hdr->done, 0u);
      advance_call(p.hdr);
    }
  }
}

// Lambda gradient: each channel's per-tile partials summed over (chunk, batch
// row) in a fixed order (16 waves take contiguous runs, then the runs in wave
// order), times sigma(lambda) and -c.
__global__ __launch_bounds__(1024) void bwd_dlam_kernel(BwdArgs p) {
  constexpr int NWR = 16;
  __shared__ float s_sum[NWR][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int ch = blockIdx.x * 64 + lane;
  const bool active = ch < p.W;
  const int strip = blockIdx.x;
  const int n_parts = p.n_chunks * p.B;
  const int per = (n_parts + NWR - 1) / NWR;
  const int k0 = wave * per;
  const int k1 = k0 + per < n_parts ? k0 + per : n_parts;
  float s = 0.0f;
  if (active) {
#pragma unroll 8
    for (int k = k0; k < k1; ++k) {
      // k = chunk * B + b: tile (chunk, b, strip)
      const size_t tile = static_cast<size_t>(k) * p.n_strips + strip;
      s += p.part[tile * 64 + lane];
    }
  }
  s_sum[wave][lane] = s;
  __syncthreads();
  if (wave == 0 && active) {
    float tot = 0.0f;
    for (int w = 0; w < NWR; ++w) tot += s_sum[w][lane];
    const float lm = p.lam[ch];
    const float sig = 1.0f / (1.0f + expf(-lm));
    p.dlam[ch] = -p.c * sig * tot;
  }
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
  // (each factor bounded before the product, so none of it can overflow)
  if (s->batch > (1LL << 24) || s->width > (1LL << 24) || s->length > (1LL << 34)) return false;
  const long long rows = ceil_div(s->width, 64) * s->batch;   // < 2^43
  if (rows >= (1LL << 31)) return false;
  const long long tiles = rows * ceil_div(s->length, 8);       // < 2^62
  if (tiles >= (1LL << 31)) return false;
  return true;
}

Geometry geometry(const rglru_shape_t* s) {
  Geometry g;
  g.io_bytes = s->io_dtype == RGLRU_IO_F32 ? 4 : 2;
  const int req = s->chunk == 0 ? 64 : s->chunk;
  // the shortest tile a request can run with in each direction (the tile
  // also depends on pointer alignment, unknown here), so the chunk counts
  // below bound those of any launch
  g.T = req > 64 ? 64 : req;
  g.Tb = req > 32 ? 32 : req;
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

// slot kinds: forward map A, map B, carry; the backward adds the partials
size_t ws_bytes(const rglru_shape_t* s, int n_chunks, int kinds) {
  return kHeaderBytes + static_cast<size_t>(kinds) * round_up(slot_words(s, n_chunks) * 8, 256);
}

size_t fwd_ws(const rglru_shape_t* s) { return ws_bytes(s, geometry(s).n_chunks_f, 3); }
size_t bwd_ws(const rglru_shape_t* s) { return ws_bytes(s, geometry(s).n_chunks_b, 4); }

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


// Workgroups of `kernel` that fit on the device at once (0 on a HIP error).
template <typename Kern>
unsigned resident_blocks(Kern kernel, int threads) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess) return 0;
  if (per_cu < 1) per_cu = 1;
  return static_cast<unsigned>(cus) * static_cast<unsigned>(per_cu);
}

// Number of workgroups of a persistent kernel: as many as fit on the device at once.
template <typename Kern>
unsigned persistent_grid(Kern kernel, int threads, unsigned n_tiles) {
  const unsigned g = resident_blocks(kernel, threads);
  return g < n_tiles ? g : n_tiles;
}

template <typename IO, int NW, int TS, bool WIDE>
rglru_status_t launch_fwd(FwdArgs a, hipStream_t stream) {
  constexpr int T = NW * TS;
  a.n_strips = static_cast<int>(ceil_div(a.W, 64));
  a.n_chunks = static_cast<int>(ceil_div(a.L, T));
  a.n_tiles = static_cast<unsigned>(a.n_chunks) * static_cast<unsigned>(a.B) * static_cast<unsigned>(a.n_strips);
  // packed sequences run their own instantiation, so the plain kernel carries
  // none of their registers
  auto kernel = a.seg != nullptr ? fwd_kernel<IO, NW, TS, WIDE, true, false> : fwd_kernel<IO, NW, TS, WIDE, false, false>;
  constexpr int threads = (NW + 4) * 64;
  const unsigned grid = persistent_grid(kernel, threads, a.n_tiles);
  if (grid == 0) return RGLRU_ERR_HIP;
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(threads), 0, stream, a);
  return launch_status();
}

// The forward with both gate projections computed inside it: bf16, 64-step
// tiles of 8 data waves (the projection's block rows of a 128-step tile would
// not fit LDS twice).
rglru_status_t launch_fused(FwdArgs a, hipStream_t stream) {
  constexpr int NW = 8, TS = 8, T = NW * TS;
  a.n_strips = static_cast<int>(ceil_div(a.W, 64));
  a.n_chunks = static_cast<int>(ceil_div(a.L, T));
  a.n_tiles = static_cast<unsigned>(a.n_chunks) * static_cast<unsigned>(a.B) * static_cast<unsigned>(a.n_strips);
  auto kernel = fwd_kernel<BF16, NW, TS, true, false, true>;
  constexpr int threads = (NW + 8) * 64;
  const unsigned grid = persistent_grid(kernel, threads, a.n_tiles);
  if (grid == 0) return RGLRU_ERR_HIP;
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(threads), 0, stream, a);
  return launch_status();
}

// Both gates' weights [nb][256 in][256 out] into the fused projection's
// fragment order (see fused_w_frag): thread (fragment, lane) gathers its 8
// inputs of one output; a wave's reads of one input row are 32 consecutive
// outputs.
__global__ __launch_bounds__(256) void w_frag_kernel(const uint16_t* w0, const uint16_t* w1, uint16_t* f0, uint16_t* f1,
                                                     long long n_frag) {
  const long long id = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  const long long frag = id >> 6;
  if (frag >= 2 * n_frag) return;
  const int g = frag >= n_frag ? 1 : 0;
  const long long fr = frag - g * n_frag;
  const int lane = static_cast<int>(id & 63);
  const int ks = static_cast<int>(fr & 15);
  const int ot = static_cast<int>((fr >> 4) & 7);
  const long long kb = fr >> 7;
  const uint16_t* src = (g ? w1 : w0) + kb * 65536 + (ks * 16 + (lane >> 5) * 8) * 256 + ot * 32 + (lane & 31);
  uint16_t v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = src[e * 256];
  uint16_t* dst = (g ? f1 : f0) + (fr * 64 + lane) * 8;
  *reinterpret_cast<u32x4*>(dst) = __builtin_bit_cast(u32x4, v);
}

// Forward tile length for a requested chunk: at most 128 steps where 2-byte
// rows are loaded 16 bytes per lane (a tile's raw words then fill 48 KiB of
// LDS, and the pipeline holds two), at most 64 otherwise.
int fwd_tile(int req, bool wide, int io_bytes) {
  const int cap = (wide && io_bytes == 2) ? 128 : 64;
  return req < cap ? req : cap;
}

// Tiles of T steps: T / 8 data waves of 8 steps each up to 64 steps, 8 data
// waves of 16 steps at 128.
template <typename IO, bool WIDE>
rglru_status_t dispatch_fwd(int T, FwdArgs a, hipStream_t stream) {
  switch (T) {
    case 8: return launch_fwd<IO, 1, 8, WIDE>(a, stream);
    case 16: return launch_fwd<IO, 2, 8, WIDE>(a, stream);
    case 32: return launch_fwd<IO, 4, 8, WIDE>(a, stream);
    case 64: return launch_fwd<IO, 8, 8, WIDE>(a, stream);
    default: break;
  }
  if constexpr (WIDE && std::is_same<IO, BF16>::value) {
    if (T == 128) return launch_fwd<IO, 8, 16, WIDE>(a, stream);
  }
  return RGLRU_ERR_UNSUPPORTED;
}

template <typename IO, int NW, bool WIDE>
rglru_status_t launch_bwd(BwdArgs a, hipStream_t stream) {
  constexpr int T = NW * kCkpt;
  a.n_strips = static_cast<int>(ceil_div(a.W, 64));
  a.n_chunks = static_cast<int>(ceil_div(a.L, T));
  a.n_tiles = static_cast<unsigned>(a.n_chunks) * static_cast<unsigned>(a.B) * static_cast<unsigned>(a.n_strips);
  auto kernel = a.seg != nullptr ? bwd_kernel<IO, NW, WIDE, true> : bwd_kernel<IO, NW, WIDE, false>;
  constexpr int threads = (NW + 4) * 64;
  const unsigned grid = persistent_grid(kernel, threads, a.n_tiles);
  if (grid == 0) return RGLRU_ERR_HIP;
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(threads), 0, stream, a);
  rglru_status_t st = launch_status();
  if (st != RGLRU_OK) return st;
  hipLaunchKernelGGL(bwd_dlam_kernel, dim3(static_cast<unsigned>(a.n_strips)), dim3(1024), 0, stream, a);
  return launch_status();
}

// Backward tile length for a requested chunk: at most 64 steps where 2-byte
// rows are loaded 16 bytes per lane (a tile's raw words then fill 32 KiB of
// LDS and the pipeline holds two), at most 32 otherwise.
int bwd_tile(int req, bool wide, int io_bytes) {
  const int cap = (wide && io_bytes == 2) ? 64 : 32;
  return req < cap ? req : cap;
}

template <typename IO, bool WIDE>
rglru_status_t dispatch_bwd(int T, BwdArgs a, hipStream_t stream) {
  switch (T) {
    case 8: return launch_bwd<IO, 1, WIDE>(a, stream);
    case 16: return launch_bwd<IO, 2, WIDE>(a, stream);
    case 32: return launch_bwd<IO, 4, WIDE>(a, stream);
    default: break;
  }
  if constexpr (WIDE && std::is_same<IO, BF16>::value) {
    if (T == 64) return launch_bwd<IO, 8, WIDE>(a, stream);
  }
  return RGLRU_ERR_UNSUPPORTED;
}

bool io_aligned(const void* p, int io_bytes) { return p == nullptr || aligned_to(p, io_bytes); }
bool f32_aligned(const void* p) { return p == nullptr || aligned_to(p, 4); }

}  // namespace
}  // namespace rglru

using namespace rglru;

// ------------------------------------------------------------------ calls

namespace {

// Packed sequences on top of a call: per-token segment words (in the
// workspace) and the per-segment states and gradients. All null for a plain
// call.
struct Packed {
  const int32_t* cu = nullptr;     // segment offsets [n + 1]
  long long n = 0;
  uint32_t* seg = nullptr;         // segment words, written by the call
  const float* h0s = nullptr;
  float* h_last_s = nullptr;
  const float* dh_last_s = nullptr;
  float* dh0s = nullptr;
};

// ------------------------------------------------------------------ packed sequences
//
// n segments packed end to end in one row of T tokens, segment s holding
// tokens [cu[s], cu[s+1]). Each segment is its own sequence: its first token
// starts from the segment's initial state (zero without one) and its last
// token's state is the segment's final state; reset tokens inside keep their
// meaning. The scan kernels read one segment word per token.

// Segment word of every token; error bit 2 if the offsets are not
// 0 = cu[0] <= cu[1] <= ... <= cu[n] = T. Invalid offsets still give every
// token a segment index below n, so nothing is addressed out of bounds.
__global__ __launch_bounds__(256) void varlen_seg_kernel(const int32_t* cu, long long n, long long T, uint32_t* seg,
                                                        Header* hdr) {
  const long long t = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  if (t < n && cu[t] > cu[t + 1]) atomicOr(&hdr->err, 4u);
  if (t == 0 && (cu[0] != 0 || static_cast<long long>(cu[n]) != T)) atomicOr(&hdr->err, 4u);
  if (t >= T) return;
  // the last segment starting at or before t (empty segments are skipped
  // over: a later segment with the same start wins)
  long long lo = 0, hi = n - 1;
  while (lo < hi) {
    const long long mid = (lo + hi + 1) >> 1;
    if (static_cast<long long>(cu[mid]) <= t) {
      lo = mid;
    } else {
      hi = mid - 1;
    }
  }
  uint32_t w = static_cast<uint32_t>(lo) & kSegId;
  if (static_cast<long long>(cu[lo]) == t) w |= kSegStart;
  if (static_cast<long long>(cu[lo + 1]) - 1 == t) w |= kSegEnd;
  seg[t] = w;
}

// Segments without tokens: final state = initial state (forward), gradient on
// the initial state = gradient on the final state (backward).
__global__ __launch_bounds__(256) void varlen_empty_kernel(const int32_t* cu, long long n, int W, const float* src,
                                                          float* dst) {
  const long long i = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n * W) return;
  const long long sgi = i / W;
  if (cu[sgi] >= cu[sgi + 1]) dst[i] = src != nullptr ? src[i] : 0.0f;
}

size_t varlen_ws(const rglru_shape_t* s) {
  const size_t f = fwd_ws(s), b = bwd_ws(s);
  return (f > b ? f : b) + round_up(static_cast<size_t>(s->length) * 4, 256);
}

// Checks shared by both directions; the segment words go after the slots.
rglru_status_t varlen_check(const rglru_shape_t* s, const int32_t* cu, long long n, void* workspace,
                            size_t workspace_bytes, Packed* pk) {
  if (!shape_ok(s) || s->batch != 1 || n < 1 || n > static_cast<long long>(kSegId) || cu == nullptr ||
      workspace == nullptr) {
    return RGLRU_ERR_INVALID_ARGUMENT;
  }
  if (!aligned_to(cu, 4) || !aligned_to(workspace, 256)) return RGLRU_ERR_MISALIGNED;
  if (workspace_bytes < varlen_ws(s)) return RGLRU_ERR_WORKSPACE_TOO_SMALL;
  const size_t f = fwd_ws(s), b = bwd_ws(s);
  pk->cu = cu;
  pk->n = n;
  pk->seg = reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + (f > b ? f : b));
  return RGLRU_OK;
}

rglru_status_t launch_seg(const rglru_shape_t* s, const Packed& pk, void* workspace, hipStream_t st) {
  const long long threads = s->length > pk.n ? s->length : pk.n;
  hipLaunchKernelGGL(varlen_seg_kernel, dim3(static_cast<unsigned>(ceil_div(threads, 256))), dim3(256), 0, st,
                     pk.cu, pk.n, static_cast<long long>(s->length), pk.seg, static_cast<Header*>(workspace));
  return launch_status();
}

rglru_status_t fwd_call(const rglru_shape_t* s, const void* x, const void* gate_x, const void* gate_a,
                        const float* lambda, const uint8_t* reset, const float* h0, void* h,
                        float* h_last, float* ckpt, void* workspace, size_t workspace_bytes,
                        void* stream, const Packed& pk) {
  if (!shape_ok(s)) return RGLRU_ERR_INVALID_ARGUMENT;
  if (!x || !gate_x || !gate_a || !lambda || !h || !workspace) return RGLRU_ERR_INVALID_ARGUMENT;
  const Geometry g = geometry(s);
  if (!io_aligned(x, g.io_bytes) || !io_aligned(gate_x, g.io_bytes) || !io_aligned(gate_a, g.io_bytes) ||
      !io_aligned(h, g.io_bytes) || !f32_aligned(lambda) || !f32_aligned(h0) || !f32_aligned(h_last) ||
      !f32_aligned(ckpt) || !aligned_to(workspace, 256)) {
    return RGLRU_ERR_MISALIGNED;
  }
  if (workspace_bytes < fwd_ws(s)) return RGLRU_ERR_WORKSPACE_TOO_SMALL;
  if (!f32_aligned(pk.h0s) || !f32_aligned(pk.h_last_s)) return RGLRU_ERR_MISALIGNED;

  if (pk.cu != nullptr) {
    const rglru_status_t r = launch_seg(s, pk, workspace, static_cast<hipStream_t>(stream));
    if (r != RGLRU_OK) return r;
  }
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
  a.seg = pk.seg;
  a.h0s = pk.h0s;
  a.h_last_s = pk.h_last_s;
  a.wt[0] = a.wt[1] = nullptr;
  a.pbias[0] = a.pbias[1] = nullptr;
  a.gout[0] = a.gout[1] = nullptr;
  a.hdr = sl.hdr;
  a.slot_a = sl.a;
  a.slot_b = sl.b;
  a.slot_h = sl.h;
  a.L = s->length;
  a.n_ckpt = g.n_ckpt;
  a.B = static_cast<int>(s->batch);
  a.W = static_cast<int>(s->width);
  a.c = s->c;
  // 16-byte loads: rows a multiple of 16 bytes, the three inputs 16-byte aligned
  const bool wide = (s->width * g.io_bytes) % 16 == 0 && aligned_to(x, 16) && aligned_to(gate_x, 16) &&
                    aligned_to(gate_a, 16) && 128LL * s->width * g.io_bytes < (1LL << 31);
  a.h_wide = (s->width * g.io_bytes) % 16 == 0 && aligned_to(h, 16);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (s->length <= kSerialMaxL) {
    const unsigned grid = static_cast<unsigned>(ceil_div(s->batch * (s->width / V), 256));
    if (s->io_dtype == RGLRU_IO_F32) {
      hipLaunchKernelGGL((fwd_serial_kernel<F32, 1>), dim3(static_cast<unsigned>(ceil_div(s->batch * s->width, 256))),
                         dim3(256), 0, st, a);
    } else if (V >= 4) {
      hipLaunchKernelGGL((fwd_serial_kernel<BF16, 4>), dim3(grid), dim3(256), 0, st, a);
    } else if (V == 2) {
      hipLaunchKernelGGL((fwd_serial_kernel<BF16, 2>), dim3(grid), dim3(256), 0, st, a);
    } else {
      hipLaunchKernelGGL((fwd_serial_kernel<BF16, 1>), dim3(grid), dim3(256), 0, st, a);
    }
    return launch_status();
  }
  const int req = s->chunk == 0 ? 128 : s->chunk;
  const int T = fwd_tile(req, wide, g.io_bytes);
  if (s->io_dtype == RGLRU_IO_F32) {
    return wide ? dispatch_fwd<F32, true>(T, a, st) : dispatch_fwd<F32, false>(T, a, st);
  }
  return wide ? dispatch_fwd<BF16, true>(T, a, st) : dispatch_fwd<BF16, false>(T, a, st);
}

rglru_status_t bwd_call(const rglru_shape_t* s, const void* x, const void* gate_x, const void* gate_a,
                        const float* lambda, const uint8_t* reset, const float* ckpt, const void* dh,
                        const float* dh_last, void* dx, void* dgate_x, void* dgate_a, float* dlambda,
                        float* dh0, void* workspace, size_t workspace_bytes, void* stream, const Packed& pk) {
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
  if (!f32_aligned(pk.h0s) || !f32_aligned(pk.dh_last_s) || !f32_aligned(pk.dh0s)) return RGLRU_ERR_MISALIGNED;
  if (pk.cu != nullptr) {
    const rglru_status_t r = launch_seg(s, pk, workspace, static_cast<hipStream_t>(stream));
    if (r != RGLRU_OK) return r;
  }

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
  a.seg = pk.seg;
  a.h0s = pk.h0s;
  a.dh_last_s = pk.dh_last_s;
  a.dh0s = pk.dh0s;
  a.hdr = sl.hdr;
  a.slot_a = sl.a;
  a.slot_b = sl.b;
  a.slot_h = sl.h;
  a.part = reinterpret_cast<float*>(sl.p);
  a.L = s->length;
  a.n_ckpt = g.n_ckpt;
  a.B = static_cast<int>(s->batch);
  a.W = static_cast<int>(s->width);
  a.c = s->c;
  // 16-byte loads: rows a multiple of 16 bytes, the four inputs 16-byte aligned
  const bool wide = (s->width * g.io_bytes) % 16 == 0 && aligned_to(x, 16) && aligned_to(gate_x, 16) &&
                    aligned_to(gate_a, 16) && aligned_to(dh, 16) && 64LL * s->width * g.io_bytes < (1LL << 31);
  a.out_wide = (s->width * g.io_bytes) % 16 == 0 && aligned_to(dx, 16) && aligned_to(dgate_x, 16) &&
               aligned_to(dgate_a, 16);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int req = s->chunk == 0 ? 64 : s->chunk;
  const int T = bwd_tile(req, wide, g.io_bytes);
  if (s->io_dtype == RGLRU_IO_F32) {
    return wide ? dispatch_bwd<F32, true>(T, a, st) : dispatch_bwd<F32, false>(T, a, st);
  }
  return wide ? dispatch_bwd<BF16, true>(T, a, st) : dispatch_bwd<BF16, false>(T, a, st);
}

}  // namespace

// ------------------------------------------------------------------ allocation-free forward
//
// rglru_fwd_scratch runs rglru_fwd with this array as its workspace. Each GPU
// the library runs on holds its own copy (zero when the code object loads)
// until the process ends. Like a caller's workspace it is left ready for the
// next call by every completed call, so it is never cleared. In host code the
// array's name is not a device address: the address of the current device's
// copy is looked up once per device and kept.
constexpr size_t kScratchBytes = RGLRU_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mu;

// The current device's copy of the scratch array, or nullptr if the runtime
// cannot give its address.
void* scratch_addr(int dev) {
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch_addr[dev].load(std::memory_order_relaxed);
  if (p == nullptr) {
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr) return nullptr;
    g_scratch_addr[dev].store(q, std::memory_order_release);
    p = q;
  }
  return p;
}
}  // namespace

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
  return fwd_call(s, x, gate_x, gate_a, lambda, reset, h0, h, h_last, ckpt, workspace, workspace_bytes, stream,
                  Packed{});
}

rglru_status_t rglru_bwd(const rglru_shape_t* s, const void* x, const void* gate_x, const void* gate_a,
                         const float* lambda, const uint8_t* reset, const float* ckpt, const void* dh,
                         const float* dh_last, void* dx, void* dgate_x, void* dgate_a, float* dlambda,
                         float* dh0, void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_call(s, x, gate_x, gate_a, lambda, reset, ckpt, dh, dh_last, dx, dgate_x, dgate_a, dlambda, dh0,
                  workspace, workspace_bytes, stream, Packed{});
}

rglru_status_t rglru_fwd_scratch(const rglru_shape_t* s, const void* x, const void* gate_x, const void* gate_a,
                                 const float* lambda, const uint8_t* reset, const float* h0, void* h,
                                 float* h_last, float* ckpt, void* stream) {
  if (!shape_ok(s)) return RGLRU_ERR_INVALID_ARGUMENT;
  if (fwd_ws(s) > kScratchBytes) return RGLRU_ERR_SCRATCH_TOO_SMALL;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return RGLRU_ERR_HIP;
  void* ws = scratch_addr(dev);
  if (ws == nullptr) return RGLRU_ERR_HIP;
  return rglru_fwd(s, x, gate_x, gate_a, lambda, reset, h0, h, h_last, ckpt, ws, kScratchBytes, stream);
}

size_t rglru_varlen_workspace_bytes(const rglru_shape_t* s, int64_t n_seqs) {
  if (!shape_ok(s) || s->batch != 1 || n_seqs < 1 || n_seqs > static_cast<int64_t>(kSegId)) return 0;
  return varlen_ws(s);
}

rglru_status_t rglru_fwd_varlen(const rglru_shape_t* s, const int32_t* cu_seqlens, int64_t n_seqs, const void* x,
                                const void* gate_x, const void* gate_a, const float* lambda, const uint8_t* reset,
                                const float* h0, void* h, float* h_last, float* ckpt, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (!x || !gate_x || !gate_a || !lambda || !h) return RGLRU_ERR_INVALID_ARGUMENT;
  if (!f32_aligned(h0) || !f32_aligned(h_last)) return RGLRU_ERR_MISALIGNED;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Packed pk;
  rglru_status_t r = varlen_check(s, cu_seqlens, n_seqs, workspace, workspace_bytes, &pk);
  if (r != RGLRU_OK) return r;
  pk.h0s = h0;
  pk.h_last_s = h_last;
  r = fwd_call(s, x, gate_x, gate_a, lambda, reset, nullptr, h, nullptr, ckpt, workspace, workspace_bytes, st, pk);
  if (r != RGLRU_OK || h_last == nullptr) return r;
  const long long n = n_seqs * s->width;
  hipLaunchKernelGGL(varlen_empty_kernel, dim3(static_cast<unsigned>(ceil_div(n, 256))), dim3(256), 0, st,
                     cu_seqlens, static_cast<long long>(n_seqs), static_cast<int>(s->width), h0, h_last);
  return launch_status();
}

rglru_status_t rglru_bwd_varlen(const rglru_shape_t* s, const int32_t* cu_seqlens, int64_t n_seqs, const void* x,
                                const void* gate_x, const void* gate_a, const float* lambda, const uint8_t* reset,
                                const float* h0, const float* ckpt, const void* dh, const float* dh_last, void* dx,
                                void* dgate_x, void* dgate_a, float* dlambda, float* dh0, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (!x || !gate_x || !gate_a || !lambda || !ckpt || !dh || !dx || !dgate_x || !dgate_a || !dlambda) {
    return RGLRU_ERR_INVALID_ARGUMENT;
  }
  if (!f32_aligned(h0) || !f32_aligned(dh_last) || !f32_aligned(dh0)) return RGLRU_ERR_MISALIGNED;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Packed pk;
  rglru_status_t r = varlen_check(s, cu_seqlens, n_seqs, workspace, workspace_bytes, &pk);
  if (r != RGLRU_OK) return r;
  pk.h0s = h0;
  pk.dh_last_s = dh_last;
  pk.dh0s = dh0;
  r = bwd_call(s, x, gate_x, gate_a, lambda, reset, ckpt, dh, nullptr, dx, dgate_x, dgate_a, dlambda, nullptr,
               workspace, workspace_bytes, st, pk);
  if (r != RGLRU_OK || dh0 == nullptr) return r;
  const long long n = n_seqs * s->width;
  hipLaunchKernelGGL(varlen_empty_kernel, dim3(static_cast<unsigned>(ceil_div(n, 256))), dim3(256), 0, st,
                     cu_seqlens, static_cast<long long>(n_seqs), static_cast<int>(s->width), dh_last, dh0);
  return launch_status();
}

size_t rglru_blockdiag_fused_fwd_workspace_bytes(const rglru_shape_t* s) {
  if (!shape_ok(s) || s->io_dtype != RGLRU_IO_BF16 || s->width % 256 != 0) return 0;
  return fwd_ws(s) + round_up(static_cast<size_t>(s->width) * 256 * 2 * 2, 256);
}

rglru_status_t rglru_blockdiag_fused_fwd(const rglru_shape_t* s, const void* x, const void* w_x, const void* b_x,
                                         const void* w_a, const void* b_a, const float* lambda, const uint8_t* reset,
                                         const float* h0, void* h, float* h_last, float* ckpt, void* gate_x,
                                         void* gate_a, void* workspace, size_t workspace_bytes, void* stream) {
  if (!shape_ok(s)) return RGLRU_ERR_INVALID_ARGUMENT;
  if (!x || !w_x || !w_a || !lambda || !h || !workspace) return RGLRU_ERR_INVALID_ARGUMENT;
  if (s->io_dtype != RGLRU_IO_BF16 || s->width % 256 != 0 || (s->chunk != 0 && s->chunk != 64) ||
      64LL * s->width * 2 >= (1LL << 31)) {
    return RGLRU_ERR_UNSUPPORTED;
  }
  const Geometry g = geometry(s);
  if (!aligned_to(x, 16) || !aligned_to(h, 16) || !aligned_to(w_x, 2) || !aligned_to(w_a, 2) ||
      !aligned_to(b_x, 2) || !aligned_to(b_a, 2) || !aligned_to(gate_x, 8) || !aligned_to(gate_a, 8) ||
      !f32_aligned(lambda) || !f32_aligned(h0) || !f32_aligned(h_last) || !f32_aligned(ckpt) ||
      !aligned_to(workspace, 256)) {
    return RGLRU_ERR_MISALIGNED;
  }
  if (workspace_bytes < rglru_blockdiag_fused_fwd_workspace_bytes(s)) return RGLRU_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const long long nb = s->width / 256;
  uint16_t* wt0 = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) + fwd_ws(s));
  uint16_t* wt1 = wt0 + nb * 65536;
  const long long n_frag = nb * 128;   // per gate: 8 output tiles x 16 input steps per block
  hipLaunchKernelGGL(w_frag_kernel, dim3(static_cast<unsigned>(ceil_div(2 * n_frag * 64, 256))), dim3(256), 0, st,
                     static_cast<const uint16_t*>(w_x), static_cast<const uint16_t*>(w_a), wt0, wt1, n_frag);
  rglru_status_t r = launch_status();
  if (r != RGLRU_OK) return r;
  const Slots sl = slots_in(workspace, slot_words(s, g.n_chunks_f));
  FwdArgs a;
  a.x = x;
  a.gx = nullptr;
  a.ga = nullptr;
  a.lam = lambda;
  a.reset = reset;
  a.h0 = h0;
  a.h = h;
  a.h_last = h_last;
  a.ckpt = ckpt;
  a.seg = nullptr;
  a.h0s = nullptr;
  a.h_last_s = nullptr;
  a.wt[0] = wt0;
  a.wt[1] = wt1;
  a.pbias[0] = static_cast<const uint16_t*>(b_x);
  a.pbias[1] = static_cast<const uint16_t*>(b_a);
  a.gout[0] = static_cast<uint16_t*>(gate_x);
  a.gout[1] = static_cast<uint16_t*>(gate_a);
  a.hdr = sl.hdr;
  a.slot_a = sl.a;
  a.slot_b = sl.b;
  a.slot_h = sl.h;
  a.L = s->length;
  a.n_ckpt = g.n_ckpt;
  a.B = static_cast<int>(s->batch);
  a.W = static_cast<int>(s->width);
  a.c = s->c;
  a.h_wide = true;
  return launch_fused(a, st);
}

const char* rglru_status_string(rglru_status_t status) {
  // A C caller may pass any int; in C++ an enum object holding a value
  // outside its enumerators' range may not be read as the enum, so its
  // bits are read as an int.
  int v = 0;
  static_assert(sizeof(status) == sizeof(v), "the status enum has the size of int");
  std::memcpy(&v, &status, sizeof(v));
  switch (v) {
    case RGLRU_OK: return "RGLRU_OK";
    case RGLRU_ERR_INVALID_ARGUMENT: return "RGLRU_ERR_INVALID_ARGUMENT: bad shape, NULL required pointer or bad enum";
    case RGLRU_ERR_MISALIGNED: return "RGLRU_ERR_MISALIGNED: a pointer is not aligned to its element size";
    case RGLRU_ERR_WORKSPACE_TOO_SMALL: return "RGLRU_ERR_WORKSPACE_TOO_SMALL";
    case RGLRU_ERR_UNSUPPORTED: return "RGLRU_ERR_UNSUPPORTED: valid request not implemented in this build";
    case RGLRU_ERR_HIP: return "RGLRU_ERR_HIP: the HIP runtime refused a launch";
    case RGLRU_ERR_SCRATCH_TOO_SMALL:
      return "RGLRU_ERR_SCRATCH_TOO_SMALL: the shape needs more workspace than RGLRU_SCRATCH_BYTES";
  }
  return "RGLRU_ERR_UNKNOWN";
}

int rglru_abi_version(void) { return RGLRU_ABI_VERSION; }

}  // extern "C"
