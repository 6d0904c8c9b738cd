// Device helpers shared by the PBSA kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pbsa.h"

namespace pbsa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// bf16 bits -> fp32 (exact)
__device__ __forceinline__ float bf2f(uint16_t x) { return __uint_as_float(uint32_t(x) << 16); }
__device__ __forceinline__ float bflo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bfhi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN)
__device__ __forceinline__ uint16_t f2bf(float f) {
  __bf16 b = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, b);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return uint32_t(f2bf(lo)) | (uint32_t(f2bf(hi)) << 16);
}

__device__ __forceinline__ void set_status(int32_t *st, int bit) {
  if (st) atomicOr(st, bit);
}

// Total order of the routing decisions (top-k over window scores, Top-C
// over block masses): larger value first, then smaller id, NaN after every
// number (NaNs among themselves by id).  order_key maps a value to a 32-bit
// key whose unsigned order is that order on the values: larger value ->
// larger key, -0 == +0, every NaN -> 1 (below all numbers, whose keys are
// >= 0x007fffff); key 0 is left for entries that take no part.  Then
// "a ranks before b" is ka > kb || (ka == kb && ida < idb), which compiles
// to compares and masks with no branches.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (f != f) return 1u;
  if ((u & 0x7fffffffu) == 0) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace pbsa
