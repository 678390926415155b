// Device-side types and helpers shared by the gfx950 SWA kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// log2(e): softmax is evaluated as exp2((s - m) * scale * log2e).
constexpr float kLog2e = 1.4426950408889634f;

// Exact widening of a bfloat16 bit pattern held in the low / high half of a
// 32-bit word.
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round two floats to bfloat16 (nearest-even, the hardware conversion) and
// pack them into one word, first argument in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  f2 v = {a, b};
  bf16x2 r = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float wave_max_xor32(float x) {
  return fmaxf(x, __shfl_xor(x, 32));
}

}  // namespace swa
