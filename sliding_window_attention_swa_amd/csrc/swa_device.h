// Device-side types and helpers shared by the gfx950 SWA kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

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

// Maximum over lanes l and l^32 of a wave (in the score layout of the MFMA
// kernels they hold the same row) with one VALU lane swap, without an LDS
// round trip.  The second input of the swap is made opaque: given the same
// value twice, the compiler folds the maximum of the two results to one of
// them.
__device__ __forceinline__ float max_lane_pair(float x) {
  uint32_t a = __float_as_uint(x), b = a;
#if defined(__HIP_DEVICE_COMPILE__)  // register constraints exist only for the GPU pass
  __asm__ volatile("" : "+v"(b));
#endif
  const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

}  // namespace swa
