// Shared device/host definitions of the convrot library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace convrot {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef unsigned short us2 __attribute__((ext_vector_type(2)));
typedef unsigned int u4 __attribute__((ext_vector_type(4)));
typedef unsigned int u2 __attribute__((ext_vector_type(2)));

// Sign vector d of the rotation (bit i set <=> d[i] = -1), i < g <= 256.
// Passed by value as a kernel argument; the host derives it from the seed.
struct SignMask {
  uint32_t w[8];
};

__host__ __device__ constexpr int ilog2(int g) { return g <= 1 ? 0 : 1 + ilog2(g >> 1); }

// Quiet NaN written to a per-row scale to mark a row that the exact
// (banded) kernel must finish. It is never a valid scale.
constexpr uint32_t kDeferredRow = 0x7FC0DEADu;

// Compute units per XCD on gfx950 (an MI355X has 8 XCDs of 32 CUs; a
// compute partition exposes whole XCDs). Workgroups of a launch are dealt to
// the XCDs round-robin.
constexpr int kCUsPerXCD = 32;
__host__ __device__ constexpr int xcd_count(int cus) {
  return cus >= 2 * kCUsPerXCD ? cus / kCUsPerXCD : 1;
}

// Bands of the exact rotation: each band spans at most kBand binades, so a
// float64 Walsh-Hadamard transform over one band is exact (see rotate.hip).
constexpr int kBand = 36;

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  const bf2 r = __builtin_convertvector((f2){lo, hi}, bf2);
  return __builtin_bit_cast(uint32_t, r);
}

// IEEE half halves of a packed pair -> fp32 (exact).
__device__ __forceinline__ float half_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(w & 0xFFFFu));
}
__device__ __forceinline__ float half_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(w >> 16));
}

// fp32 -> IEEE half bits, round to nearest even (overflow to inf).
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const h2 r = __builtin_convertvector((f2){lo, hi}, h2);
  return __builtin_bit_cast(uint32_t, r);
}

// The 16-bit format chosen at compile time: half when F16, else bf16.
template <bool F16>
__device__ __forceinline__ float lo16(uint32_t w) { return F16 ? half_lo(w) : bf16lo(w); }
template <bool F16>
__device__ __forceinline__ float hi16(uint32_t w) { return F16 ? half_hi(w) : bf16hi(w); }
template <bool F16>
__device__ __forceinline__ uint32_t pack16x2(float lo, float hi) {
  return F16 ? pack_f16x2(lo, hi) : pack_bf16x2(lo, hi);
}

}  // namespace convrot
