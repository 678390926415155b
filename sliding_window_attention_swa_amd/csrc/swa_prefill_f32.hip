// Sliding-window attention prefill in IEEE fp32 (vector ALU, full-precision
// products: the fp32 workloads are held to an absolute error of 1e-5).
//
// Same definition as the bf16 kernel (robocikowo glossary "Sliding Window
// Attention", opening definition; Ultralytics glossary, section "Come cresce
// la finestra con la profondita"): each query row takes the softmax of its
// in-window logits only.  16 lanes share one query row, each holding d/16
// dims; a row walks exactly the keys of its own window, one key at a time,
// with a running maximum and sum.
//
// Chunked prefill (MODE 2): T is the chunk length and row i is position
// p + i of its sequence; its keys r = j - p in [max(-p, i-W+1), i] come from
// ring slot (p + r) mod W when r < 0 (Ultralytics ring-buffer paragraph) and
// from chunk row r otherwise.
//
// Dilated windows (dil > 1; aivaro answer 629, section 4.2): the row takes
// every dil-th key, j = i - m * dil for m in the plain window's offsets.
//
// Global tokens (MODES 5 causal, 6 symmetric; aivaro section 4.3): after its
// window (dilated when dil > 1) the row also takes each global key outside
// the window (not after the row when causal).  The global rows themselves
// are written afterwards by the split-K pass of swa_ring.hip.

#include "swa_device.h"
#include "swa_launch.h"

namespace swa {
namespace {

constexpr int kRowsPerBlock = 16;
constexpr int kLanesPerRow = 16;

// MODE: 0 causal, 1 symmetric, 2 causal chunk continuing a ring cache
// (kring/vring/pos/hkv_seq are used by MODE 2 only), 5 causal and 6
// symmetric window plus the ngl global keys at gpos.  dil: key stride of a
// dilated window in MODES 0, 1, 5 and 6 (1 otherwise).
template <int D, int MODE>
__global__ __launch_bounds__(256) void prefill_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ out, int T, int W, int Hq, int Hkv, float scale, int n_rowblocks,
    const float* __restrict__ kring, const float* __restrict__ vring,
    const int32_t* __restrict__ pos, int hkv_seq, int dil, const int32_t* __restrict__ gpos,
    int ngl) {
  constexpr int DPL = D / kLanesPerRow;
  constexpr bool kCausal = MODE != 1 && MODE != 6;
  const int h = blockIdx.x / n_rowblocks;
  const int i = (blockIdx.x % n_rowblocks) * kRowsPerBlock + threadIdx.x / kLanesPerRow;
  const int c = threadIdx.x % kLanesPerRow;
  if (i >= T) return;  // whole 16-lane groups leave together
  const int kvh = h / (Hq / Hkv);
  const float* qrow = q + ((size_t)h * T + i) * D + c * DPL;
  const float* kh = k + (size_t)kvh * T * D + c * DPL;
  const float* vh = v + (size_t)kvh * T * D + c * DPL;

  float* orow = out + ((size_t)h * T + i) * D + c * DPL;
  int pstart = 0;  // chunk mode: position of the chunk's first token
  if constexpr (MODE == 2) {
    pstart = pos[kvh / hkv_seq];
    if (pstart < 0) {  // inactive sequence: zero rows
#pragma unroll
      for (int e = 0; e < DPL; ++e) orow[e] = 0.f;
      return;
    }
  }

  float qv[DPL], acc[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) {
    qv[e] = qrow[e];
    acc[e] = 0.f;
  }
  int lo, hi;
  if (MODE == 2) {
    lo = max(-pstart, i - W + 1);
    hi = i;
  } else if (kCausal) {
    lo = i - dil * min(W - 1, i / dil);
    hi = i;
  } else {
    lo = i - dil * min(W / 2, i / dil);
    hi = i + dil * min(W / 2, (T - 1 - i) / dil);
  }
  // chunk mode: ring slot of key lo (pstart + lo >= 0), advanced with the key
  unsigned slot = 0;
  const float* krh = nullptr;
  const float* vrh = nullptr;
  if constexpr (MODE == 2) {
    slot = (unsigned)(pstart + lo) % (unsigned)W;
    krh = kring + (size_t)kvh * W * D + c * DPL;
    vrh = vring + (size_t)kvh * W * D + c * DPL;
  }
  float m = -INFINITY, l = 0.f;
  // one key: score, running maximum and sum, accumulate its value row
  auto visit = [&](const float* kr, const float* vr) {
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) s = fmaf(qv[e], kr[e], s);
#pragma unroll
    for (int off = kLanesPerRow / 2; off > 0; off >>= 1) s += __shfl_xor(s, off, kLanesPerRow);
    s *= scale;
    const float m_new = fmaxf(m, s);
    const float alpha = expf(m - m_new);  // m = -inf on the first key: 0
    const float p = expf(s - m_new);
    l = l * alpha + p;
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[e] = fmaf(p, vr[e], acc[e] * alpha);
    m = m_new;
  };
  for (int j = lo; j <= hi; j += dil) {
    const float* kr;
    const float* vr;
    if (MODE == 2 && j < 0) {  // a ring position
      kr = krh + (size_t)slot * D;
      vr = vrh + (size_t)slot * D;
      slot = slot + 1 == (unsigned)W ? 0u : slot + 1;
    } else {
      kr = kh + (size_t)j * D;
      vr = vh + (size_t)j * D;
    }
    visit(kr, vr);
  }
  if constexpr (MODE == 5 || MODE == 6) {
    for (int t = 0; t < ngl; ++t) {
      const int gp = gpos[t];
      const int diff = i - gp;
      // in the (dilated) window: on the row's grid, within the window's offsets
      const int m = diff / dil;
      const bool in_window = diff == m * dil &&
                             (kCausal ? (m >= 0 && m < W) : (m >= -(W / 2) && m <= W / 2));
      if (gp < 0 || gp >= T || in_window || (kCausal && diff < 0)) continue;
      visit(kh + (size_t)gp * D, vh + (size_t)gp * D);
    }
  }
  const float inv = 1.0f / l;
#pragma unroll
  for (int e = 0; e < DPL; ++e) orow[e] = acc[e] * inv;
}

template <int D, int MODE>
hipError_t launch(const void* q, const void* k, const void* v, void* out, int T, int W, int Hq,
                  int Hkv, float scale, int dil, hipStream_t stream) {
  const int n_rowblocks = (T + kRowsPerBlock - 1) / kRowsPerBlock;
  const long long nwg = (long long)n_rowblocks * Hq;
  hipLaunchKernelGGL((prefill_f32_kernel<D, MODE>), dim3((unsigned)nwg),
                     dim3(kRowsPerBlock * kLanesPerRow), 0,
                     stream, static_cast<const float*>(q), static_cast<const float*>(k),
                     static_cast<const float*>(v), static_cast<float*>(out), T, W, Hq, Hkv,
                     scale, n_rowblocks, static_cast<const float*>(nullptr),
                     static_cast<const float*>(nullptr), static_cast<const int32_t*>(nullptr), 1,
                     dil, static_cast<const int32_t*>(nullptr), 0);
  return hipGetLastError();
}

template <int D>
hipError_t launch_chunk(const void* q, const void* k, const void* v, const void* k_ring,
                        const void* v_ring, const int32_t* pos, void* out, int B, int n, int W,
                        int Hq, int Hkv, float scale, hipStream_t stream) {
  const int n_rowblocks = (n + kRowsPerBlock - 1) / kRowsPerBlock;
  const long long nwg = (long long)n_rowblocks * Hq * B;
  hipLaunchKernelGGL((prefill_f32_kernel<D, 2>), dim3((unsigned)nwg),
                     dim3(kRowsPerBlock * kLanesPerRow), 0, stream, static_cast<const float*>(q),
                     static_cast<const float*>(k), static_cast<const float*>(v),
                     static_cast<float*>(out), n, W, Hq * B, Hkv * B, scale, n_rowblocks,
                     static_cast<const float*>(k_ring), static_cast<const float*>(v_ring), pos,
                     Hkv, 1, static_cast<const int32_t*>(nullptr), 0);
  return hipGetLastError();
}

template <int D, int MODE>
hipError_t launch_global(const void* q, const void* k, const void* v, void* out, int T, int W,
                         int Hq, int Hkv, float scale, const int32_t* gpos, int ngl, int dil,
                         hipStream_t stream) {
  const int n_rowblocks = (T + kRowsPerBlock - 1) / kRowsPerBlock;
  const long long nwg = (long long)n_rowblocks * Hq;
  hipLaunchKernelGGL((prefill_f32_kernel<D, MODE>), dim3((unsigned)nwg),
                     dim3(kRowsPerBlock * kLanesPerRow), 0, stream, static_cast<const float*>(q),
                     static_cast<const float*>(k), static_cast<const float*>(v),
                     static_cast<float*>(out), T, W, Hq, Hkv, scale, n_rowblocks,
                     static_cast<const float*>(nullptr), static_cast<const float*>(nullptr),
                     static_cast<const int32_t*>(nullptr), 1, dil, gpos, ngl);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_global_window_f32(const void* q, const void* k, const void* v,
                                            void* out, int T, int W, int Hq, int Hkv, int d,
                                            int mode, float scale, const int32_t* gpos, int ngl,
                                            int dil, hipStream_t stream) {
  if (mode == 0) {
    if (d == 32) return launch_global<32, 5>(q, k, v, out, T, W, Hq, Hkv, scale, gpos, ngl, dil, stream);
    if (d == 64) return launch_global<64, 5>(q, k, v, out, T, W, Hq, Hkv, scale, gpos, ngl, dil, stream);
    return launch_global<128, 5>(q, k, v, out, T, W, Hq, Hkv, scale, gpos, ngl, dil, stream);
  }
  if (d == 32) return launch_global<32, 6>(q, k, v, out, T, W, Hq, Hkv, scale, gpos, ngl, dil, stream);
  if (d == 64) return launch_global<64, 6>(q, k, v, out, T, W, Hq, Hkv, scale, gpos, ngl, dil, stream);
  return launch_global<128, 6>(q, k, v, out, T, W, Hq, Hkv, scale, gpos, ngl, dil, stream);
}

hipError_t launch_prefill_chunk_f32(const void* q, const void* k, const void* v,
                                    const void* k_ring, const void* v_ring, const int32_t* pos,
                                    void* out, int B, int n, int W, int Hq, int Hkv, int d,
                                    float scale, hipStream_t stream) {
  if (d == 32) return launch_chunk<32>(q, k, v, k_ring, v_ring, pos, out, B, n, W, Hq, Hkv, scale, stream);
  if (d == 64) return launch_chunk<64>(q, k, v, k_ring, v_ring, pos, out, B, n, W, Hq, Hkv, scale, stream);
  return launch_chunk<128>(q, k, v, k_ring, v_ring, pos, out, B, n, W, Hq, Hkv, scale, stream);
}

hipError_t launch_prefill_dilated_f32(const void* q, const void* k, const void* v, void* out,
                                      int T, int W, int Hq, int Hkv, int d, int mode, float scale,
                                      int dil, hipStream_t stream) {
  if (mode == 0) {
    if (d == 32) return launch<32, 0>(q, k, v, out, T, W, Hq, Hkv, scale, dil, stream);
    if (d == 64) return launch<64, 0>(q, k, v, out, T, W, Hq, Hkv, scale, dil, stream);
    return launch<128, 0>(q, k, v, out, T, W, Hq, Hkv, scale, dil, stream);
  }
  if (d == 32) return launch<32, 1>(q, k, v, out, T, W, Hq, Hkv, scale, dil, stream);
  if (d == 64) return launch<64, 1>(q, k, v, out, T, W, Hq, Hkv, scale, dil, stream);
  return launch<128, 1>(q, k, v, out, T, W, Hq, Hkv, scale, dil, stream);
}

hipError_t launch_prefill_f32(const void* q, const void* k, const void* v, void* out, int T,
                              int W, int Hq, int Hkv, int d, int mode, float scale,
                              hipStream_t stream) {
  return launch_prefill_dilated_f32(q, k, v, out, T, W, Hq, Hkv, d, mode, scale, 1, stream);
}

}  // namespace swa
