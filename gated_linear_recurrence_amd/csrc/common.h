// Internal helpers shared by the HIP translation units of librglru.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "rglru.h"

namespace rglru {

using u64 = unsigned long long;

inline bool aligned_to(const void* p, size_t bytes) {
  return (reinterpret_cast<uintptr_t>(p) % bytes) == 0;
}

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline size_t round_up(size_t a, size_t b) { return (a + b - 1) / b * b; }

// Maps the state of the most recent launch to a status.
inline rglru_status_t launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? RGLRU_OK : RGLRU_ERR_HIP;
}

// bf16 <-> f32. Stored bf16 values are bit patterns; conversion to f32 is
// exact, conversion from f32 rounds to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float lo, float hi) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  f2 v = {lo, hi};
  b2 r = __builtin_convertvector(v, b2);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return static_cast<uint16_t>(f32x2_to_bf16x2(f, 0.0f) & 0xFFFFu);
}

// Gated delta rule checkpoints: the state entering every 8th token of each sequence, per value
// head. The first slot of sequence n is n ceil(T / 8) for B rows of T tokens, else
// floor(start / 8) + n for packed sequences (each adds at most one partial interval, so for
// ordered offsets the sequences' slots do not overlap, and clamped offsets stay below
// ceil(T / 8) + N).
constexpr int kDeltaCkpt = 8;
__host__ __device__ __forceinline__ int64_t delta_ckpt_base(bool packed, int64_t T, int n, int64_t start) {
  return packed ? start / kDeltaCkpt + n : (int64_t)n * ((T + kDeltaCkpt - 1) / kDeltaCkpt);
}
__host__ __device__ __forceinline__ int64_t delta_ckpt_slots(bool packed, int64_t T, int64_t B, int64_t n_seqs) {
  return packed ? (T + kDeltaCkpt - 1) / kDeltaCkpt + n_seqs : B * ((T + kDeltaCkpt - 1) / kDeltaCkpt);
}

}  // namespace rglru
