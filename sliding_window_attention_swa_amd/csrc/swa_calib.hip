// Calibration kernels: what this chip sustains on the two resources the
// attention kernels are bound by, measured on the same GPU as they are.  They
// compute nothing of the attention method.
//
//   * matrix cores: a loop of v_mfma_f32_32x32x16_bf16 on random bf16
//     operands (the chip lowers its clock under random-data matrix load, so
//     constant or zero operands would overstate what attention can reach);
//   * HBM: a streaming read of a buffer larger than the Infinity Cache with
//     16-byte non-temporal loads, several in flight per lane;
//   * the vector ALU: the issue rate of fp32 FMAs and of v_exp_f32 (the
//     softmax's exponential), sixteen independent chains per lane.

#include "swa_device.h"
#include "swa_launch.h"

namespace swa {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Each lane holds four A and four B fragments (16 bytes each) from the
// operand buffer and rotates through them, so consecutive products see
// different data; four independent accumulator chains per wave.
__global__ __launch_bounds__(256) void calib_mfma_kernel(const u32x4* __restrict__ ops, int nfrag,
                                                         float* __restrict__ sink, int iters) {
  const int gid = blockIdx.x * 256 + threadIdx.x;
  u32x4 a[4], b[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    a[s] = ops[(8 * gid + s) % nfrag];
    b[s] = ops[(8 * gid + 4 + s) % nfrag];
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[s]), __builtin_bit_cast(bf16x8, b[s]), c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, b[s]), __builtin_bit_cast(bf16x8, a[(s + 1) & 3]), c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[(s + 2) & 3]), __builtin_bit_cast(bf16x8, b[(s + 1) & 3]), c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, b[(s + 3) & 3]), __builtin_bit_cast(bf16x8, a[(s + 3) & 3]), c3, 0, 0, 0);
    }
  }
  float t = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) t += c0[j] + c1[j] + c2[j] + c3[j];
  sink[gid] = t;  // keeps the products live
}

// Workgroup w reads 16-byte vectors [w * per_wg, min((w + 1) * per_wg, n16))
// with kUnroll loads in flight per lane; the XOR of everything read is stored
// so that the loads stay live.
constexpr int kUnroll = 8;

__global__ __launch_bounds__(256) void calib_read_kernel(const u32x4* __restrict__ src, size_t n16,
                                                         size_t per_wg, unsigned* __restrict__ sink) {
  const size_t lo = (size_t)blockIdx.x * per_wg;
  const size_t hi = lo + per_wg < n16 ? lo + per_wg : n16;
  unsigned acc = 0;
  size_t i = lo + threadIdx.x;
  for (; i + (size_t)256 * (kUnroll - 1) < hi; i += (size_t)256 * kUnroll) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + (size_t)256 * u);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < hi; i += 256) {  // the chunk's tail
    const u32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  sink[(size_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

// OP 0: x = fma(x, 0.999, 0.001); OP 1: x = -exp2(x).  Both chains stay in
// [-1.1, 1] from the starting values below, so no lane meets a special value.
template <int OP>
__global__ __launch_bounds__(256) void calib_vector_kernel(float* __restrict__ sink, int iters) {
  const int gid = blockIdx.x * 256 + threadIdx.x;
  float x[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) x[j] = -1.0e-3f * (float)((threadIdx.x + 16 * j) & 1023);
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if constexpr (OP == 0) {
        x[j] = fmaf(x[j], 0.999f, 0.001f);
      } else {
        x[j] = -__builtin_amdgcn_exp2f(x[j]);
      }
    }
  }
  float t = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) t += x[j];
  sink[gid] = t;  // keeps the chains live
}

}  // namespace

hipError_t launch_calib_vector(int op, float* sink, int n_wg, int iters, hipStream_t stream) {
  if (op == 0) {
    hipLaunchKernelGGL(calib_vector_kernel<0>, dim3((unsigned)n_wg), dim3(256), 0, stream, sink, iters);
  } else {
    hipLaunchKernelGGL(calib_vector_kernel<1>, dim3((unsigned)n_wg), dim3(256), 0, stream, sink, iters);
  }
  return hipGetLastError();
}

hipError_t launch_calib_mfma(const void* ops, int nfrag, float* sink, int n_wg, int iters,
                             hipStream_t stream) {
  hipLaunchKernelGGL(calib_mfma_kernel, dim3((unsigned)n_wg), dim3(256), 0, stream,
                     static_cast<const u32x4*>(ops), nfrag, sink, iters);
  return hipGetLastError();
}

hipError_t launch_calib_read(const void* src, size_t n16, unsigned* sink, int n_wg,
                             hipStream_t stream) {
  const size_t per_wg = (n16 + n_wg - 1) / n_wg;
  hipLaunchKernelGGL(calib_read_kernel, dim3((unsigned)n_wg), dim3(256), 0, stream,
                     static_cast<const u32x4*>(src), n16, per_wg, sink);
  return hipGetLastError();
}

}  // namespace swa
