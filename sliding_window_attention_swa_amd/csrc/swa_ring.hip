// Ring-buffer KV cache (append) and split-K windowed decode on gfx950.
//
// Ring (Ultralytics glossary "Sliding Window Attention", ring-buffer paragraph
// of "Come cresce la finestra con la profondita"; robocikowo glossary, rolling
// KV buffer entry): each sequence keeps W slots per KV head, position i is
// stored in slot i mod W and overwrites the oldest entry, so the cache never
// grows past W rows ("Sliding-window and hybrid attention", "Check yourself").
//
// Decode ("Sliding-window and hybrid attention", "Walking through it"): the
// query at position p reads only the window [max(0, p-W+1), p], i.e. the valid
// slots [0, min(p+1, W)); softmax does not depend on the order of the keys,
// so the slots are read in storage order.  The read of the ring dominates, so
// the kernel is organised for HBM bandwidth:
//   * grid = (sequence, KV head, query-head chunk, slot split); every K/V row
//     of a KV head is read once for all the query heads of its group;
//   * each row is read with 16-byte non-temporal loads by d/8 (bf16)
//     consecutive lanes, so a wave load covers whole rows and is fully
//     coalesced; eight loads of K and eight of V are in flight per lane;
//   * the ring is split into slot chunks only as far as needed to fill the
//     GPU; with one chunk the pass writes the output itself;
//   * q.k uses packed bf16 dot products; the sum over the lanes of a row is
//     finished with DPP row permutations (no LDS);
//   * every lane-row group keeps its own running maximum / sum (rescaled only
//     when the maximum grows by more than 2^8), merged once per workgroup
//     through LDS; a small second kernel merges the splits with the usual
//     log-sum-exp rule and writes the output.
//
// In fp32 the same two kernels also write the rows of global tokens (aivaro
// answer 629, section 4.3: a global token attends to every token): with
// GR != 0 a workgroup takes NQ (global row t, query head) pairs of one KV
// head, so they share every K/V read; the query of a pair is row gpos[t] of
// the prefill queries, and the linear K/V of the sequence serve as a ring of
// T slots of which gpos[t] + 1 (causal, GR = 1) or all T (symmetric, GR = 2)
// are valid.  In bf16 those rows are computed on the matrix cores
// (swa_prefill_bf16.hip) in the same partial layout, and the merge kernel's
// GR = 1 instantiation writes them (launch_global_combine).

#include <mutex>

#include "swa_device.h"
#include "swa_launch.h"

namespace swa {
namespace {

constexpr float kRescaleThreshold = 8.0f;
constexpr float kNegBig = -1.0e30f;
constexpr int kDecodeThreads = 256;
constexpr int kDecodeWaves = kDecodeThreads / 64;
// Measured choices:
//   kUnroll         K and V rows in flight per lane
//   kDecodeItems    (row, split) items a decode launch aims at before it
//                   stops splitting the ring
//   kGlobalItems    the same for the fp32 global-row pass
//   kGlobalNQ       (global row, head) pairs per workgroup of that pass
//   kCombineUnroll  splits in flight in the merge of many-split rows
//   kGlobalNT       non-temporal loads in the global-row pass (off: the
//                   window pass has just read those rows)
constexpr int kUnroll = 8;
constexpr int kDecodeItems = 2048;
constexpr int kGlobalItems = 2048;
constexpr int kGlobalNQ = 4;
constexpr int kCombineUnroll = 8;
constexpr bool kGlobalNT = false;

// ------------------------------------------------------------------ append

__global__ __launch_bounds__(256) void append_kernel(uint4* __restrict__ k_ring,
                                                     uint4* __restrict__ v_ring,
                                                     const int32_t* __restrict__ pos,
                                                     const uint4* __restrict__ k_new,
                                                     const uint4* __restrict__ v_new, int Hkv,
                                                     int W, int cpr, long long total) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const long long bh = idx / cpr;
  const int c = (int)(idx % cpr);
  const int b = (int)(bh / Hkv);
  const int p = pos[b];
  if (p < 0) return;
  const long long dst = (bh * W + (p % W)) * cpr + c;
  k_ring[dst] = k_new[idx];
  v_ring[dst] = v_new[idx];
}

// Append n consecutive tokens per sequence: token i goes to slot
// (pos + i) mod W.  Only the last min(n, W) tokens are written (n single
// appends in order would overwrite the earlier ones); they map to distinct
// slots, so no two threads write the same row.  One thread per 16 bytes; a
// row is 2^log_cpr such chunks, and the index space (total < 2^31) is split
// with a mask, a shift and two 32-bit divisions.
__global__ __launch_bounds__(256) void append_chunk_kernel(
    uint4* __restrict__ k_ring, uint4* __restrict__ v_ring, const int32_t* __restrict__ pos,
    const uint4* __restrict__ k, const uint4* __restrict__ v, int Hkv, int n, int n0, int W,
    int log_cpr, unsigned total) {
  const unsigned idx = blockIdx.x * 256u + threadIdx.x;
  if (idx >= total) return;
  const unsigned c = idx & ((1u << log_cpr) - 1u);
  const unsigned t = idx >> log_cpr;  // (sequence x KV head, token) row
  const unsigned m = (unsigned)(n - n0);
  const unsigned bh = t / m;
  const int i = n0 + (int)(t - bh * m);
  const int p = pos[bh / (unsigned)Hkv];
  if (p < 0) return;
  const unsigned slot = ((unsigned)p + (unsigned)i) % (unsigned)W;
  const size_t dst = (((size_t)bh * W + slot) << log_cpr) + c;
  const size_t src = (((size_t)bh * n + i) << log_cpr) + c;
  k_ring[dst] = k[src];
  v_ring[dst] = v[src];
}

// --------------------------------------------------------------- helpers

template <typename E>
struct Elem;
template <>
struct Elem<__bf16> {
  static constexpr int PER16 = 8;
  __device__ static void widen(const uint4& raw, float* f) {
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[2 * e] = bf16lo(w[e]);
      f[2 * e + 1] = bf16hi(w[e]);
    }
  }
  __device__ static void store(__bf16* dst, float x) { *dst = (__bf16)x; }
  // acc + sum of the 8 products of two 16-byte rows (packed bf16 dot2)
  __device__ static float dot(const uint4& a, const uint4& b, float acc) {
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, a.x), __builtin_bit_cast(b2, b.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, a.y), __builtin_bit_cast(b2, b.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, a.z), __builtin_bit_cast(b2, b.z), acc, false);
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, a.w), __builtin_bit_cast(b2, b.w), acc, false);
  }
};
template <>
struct Elem<float> {
  static constexpr int PER16 = 4;
  __device__ static void widen(const uint4& raw, float* f) {
    f[0] = __uint_as_float(raw.x);
    f[1] = __uint_as_float(raw.y);
    f[2] = __uint_as_float(raw.z);
    f[3] = __uint_as_float(raw.w);
  }
  __device__ static void store(float* dst, float x) { *dst = x; }
  __device__ static float dot(const uint4& a, const uint4& b, float acc) {
    acc = fmaf(__uint_as_float(a.x), __uint_as_float(b.x), acc);
    acc = fmaf(__uint_as_float(a.y), __uint_as_float(b.y), acc);
    acc = fmaf(__uint_as_float(a.z), __uint_as_float(b.z), acc);
    return fmaf(__uint_as_float(a.w), __uint_as_float(b.w), acc);
  }
};

// Sum over aligned groups of N lanes (N in {4, 8, 16, 32}); every lane of the
// group receives the total.  DPP quad permutations and row mirrors stay on
// the vector ALU.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));  // xor 1
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));  // xor 2
  if (N >= 8)
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false));  // mirror in 8
  if (N >= 16)
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x140, 0xF, 0xF, false));  // mirror in 16
  if (N >= 32) x += __shfl_xor(x, 16);
  return x;
}

// 16-byte load marked non-temporal: each ring row is read exactly once per
// decode, so it should not displace reusable lines from the caches.
template <typename E>
__device__ __forceinline__ uint4 stream_load(const E* p) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(x[0], x[1], x[2], x[3]);
}

// ------------------------------------------------------------ split pass

// GR: 0 decode, 1 / 2 rows of causal / symmetric global tokens, 3 decode
// whose every split writes its partial (slot split of S + 1 per row; the
// last slot holds the attention sinks' partial), 4 decode of one split with
// the attention sinks before the window (k_sink / v_sink) taken first in the
// same online softmax, writing the output itself
template <int GR>
constexpr bool kRows = GR == 1 || GR == 2;

template <typename E, int D, int NQ, int GR>
__global__ __launch_bounds__(kDecodeThreads) void decode_split_kernel(
    const E* __restrict__ q, const E* __restrict__ k_ring, const E* __restrict__ v_ring,
    const int32_t* __restrict__ pos, E* __restrict__ out, float* __restrict__ ws_acc,
    float* __restrict__ ws_m, float* __restrict__ ws_l, int Hq, int Hkv, int W, float scale_log2,
    int S, int chunk, int n_hchunks, int n_pairs, const E* __restrict__ k_sink,
    const E* __restrict__ v_sink, int n_sink) {
  // GR != 0: pos holds the global positions, W is the sequence length and
  // pair pi = hc * NQ + hq (of n_pairs = global rows * group size) is global
  // row pi / G with query head kvh * G + pi % G
  constexpr int EPL = Elem<E>::PER16;  // elements per 16-byte load
  constexpr int LPR = D / EPL;         // lanes per ring row
  constexpr int RPW = 64 / LPR;        // rows per wave load
  constexpr int NSTATE = kDecodeWaves * RPW;
  constexpr int STEP = kDecodeWaves * RPW * kUnroll;  // rows per workgroup step

  __shared__ float sm_acc[NQ][NSTATE][D];
  __shared__ float sm_m[NQ][NSTATE];
  __shared__ float sm_l[NQ][NSTATE];

  int id = blockIdx.x;
  const int split = id % S;
  id /= S;
  const int hc = id % n_hchunks;
  id /= n_hchunks;
  const int kvh = id % Hkv;
  const int b = id / Hkv;
  const int G = Hq / Hkv;
  const int h0 = kvh * G + hc * NQ;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int rg = lane / LPR;
  const int li = lane % LPR;

  const int p = pos[b];
  int nvalid;
  int gph[NQ], hh[NQ], s1h[NQ];  // global rows: each pair's position, head, key end
  if constexpr (kRows<GR>) {
    nvalid = 0;
#pragma unroll
    for (int hq = 0; hq < NQ; ++hq) {
      const int pi = hc * NQ + hq;
      const int gp = pi < n_pairs ? pos[pi / G] : -1;
      const bool ok = gp >= 0 && gp < W;  // positions outside the sequence are ignored
      gph[hq] = ok ? gp : -1;
      hh[hq] = kvh * G + pi % G;
      s1h[hq] = ok ? (GR == 1 ? gp + 1 : W) : 0;
      nvalid = max(nvalid, s1h[hq]);
    }
    if (nvalid == 0) return;  // no valid pair (uniform over the workgroup)
  } else {
    nvalid = p < 0 ? 0 : (p >= W ? W : p + 1);
  }
  const int s0 = split * chunk;
  const int s1 = min(s0 + chunk, nvalid);
  if constexpr (kRows<GR>) {
#pragma unroll
    for (int hq = 0; hq < NQ; ++hq) s1h[hq] = min(s0 + chunk, s1h[hq]);
  }

  uint4 qraw[NQ];  // this lane's EPL query elements of each head, as stored
#pragma unroll
  for (int hq = 0; hq < NQ; ++hq) {
    if constexpr (kRows<GR>) {  // row gph of the head's prefill queries
      qraw[hq] = gph[hq] < 0 ? make_uint4(0, 0, 0, 0)
                             : *reinterpret_cast<const uint4*>(q + ((size_t)hh[hq] * W + gph[hq]) * D + li * EPL);
    } else {
      qraw[hq] = *reinterpret_cast<const uint4*>(q + ((size_t)b * Hq + h0 + hq) * D + li * EPL);
    }
  }
  float m[NQ], l[NQ], acc[NQ][EPL];
#pragma unroll
  for (int hq = 0; hq < NQ; ++hq) {
    m[hq] = kNegBig;
    l[hq] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[hq][e] = 0.f;
  }

  size_t ring_off;
  if constexpr (kRows<GR>) {  // the sequence's linear K/V
    ring_off = (size_t)kvh * (size_t)W * D + li * EPL;
  } else {
    ring_off = ((size_t)b * Hkv + kvh) * (size_t)W * D + li * EPL;
  }
  const E* kb = k_ring + ring_off;
  const E* vb = v_ring + ring_off;

  // one workgroup step: rows base .. base + STEP - 1 (those below lim) of the
  // rows at kbp / vbp
  auto step = [&](const E* kbp, const E* vbp, int base, int lim) __attribute__((always_inline)) {
    uint4 kraw[kUnroll], vraw[kUnroll];
    bool valid[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int r = base + (u * kDecodeWaves + wave) * RPW + rg;
      valid[u] = r < lim;
      if (valid[u]) {
        if constexpr (kRows<GR> && !kGlobalNT) {  // rows the windowed pass just read
          kraw[u] = *reinterpret_cast<const uint4*>(kbp + (size_t)r * D);
          vraw[u] = *reinterpret_cast<const uint4*>(vbp + (size_t)r * D);
        } else {
          kraw[u] = stream_load(kbp + (size_t)r * D);
          vraw[u] = stream_load(vbp + (size_t)r * D);
        }
      } else {
        kraw[u] = make_uint4(0, 0, 0, 0);
        vraw[u] = make_uint4(0, 0, 0, 0);
      }
    }
    float sc[kUnroll][NQ];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
#pragma unroll
      for (int hq = 0; hq < NQ; ++hq) sc[u][hq] = Elem<E>::dot(kraw[u], qraw[hq], 0.f);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
#pragma unroll
      for (int hq = 0; hq < NQ; ++hq) {
        const float s = group_sum<LPR>(sc[u][hq]) * scale_log2;
        if constexpr (kRows<GR>) {  // each pair has its own key range
          const int r = base + (u * kDecodeWaves + wave) * RPW + rg;
          sc[u][hq] = r < s1h[hq] ? s : -INFINITY;
        } else {
          sc[u][hq] = valid[u] ? s : -INFINITY;
        }
      }
    }
    float vf[kUnroll][EPL];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) Elem<E>::widen(vraw[u], vf[u]);
#pragma unroll
    for (int hq = 0; hq < NQ; ++hq) {
      float mx = sc[0][hq];
#pragma unroll
      for (int u = 1; u < kUnroll; ++u) mx = fmaxf(mx, sc[u][hq]);
      if (mx > m[hq] + kRescaleThreshold) {
        const float alpha = __builtin_amdgcn_exp2f(m[hq] - mx);
        m[hq] = mx;
        l[hq] *= alpha;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[hq][e] *= alpha;
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const float pr = __builtin_amdgcn_exp2f(sc[u][hq] - m[hq]);
        l[hq] += pr;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[hq][e] = fmaf(pr, vf[u][e], acc[hq][e]);
      }
    }
  };
  if constexpr (GR == 4) {  // the sinks before the window, ahead of the ring's rows
    const int ns = p < 0 ? 0 : min(n_sink, max(0, p - W + 1));
    const size_t sink_off = ((size_t)b * Hkv + kvh) * (size_t)n_sink * D + li * EPL;
    for (int base = 0; base < ns; base += STEP) step(k_sink + sink_off, v_sink + sink_off, base, ns);
  }
  for (int base = s0; base < s1; base += STEP) step(kb, vb, base, s1);

  // ---- merge the NSTATE lane-row states of this workgroup
  const int st = wave * RPW + rg;
#pragma unroll
  for (int hq = 0; hq < NQ; ++hq) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) sm_acc[hq][st][li * EPL + e] = acc[hq][e];
    if (li == 0) {
      sm_m[hq][st] = m[hq];
      sm_l[hq][st] = l[hq];
    }
  }
  __syncthreads();
  for (int idx = tid; idx < NQ * D; idx += kDecodeThreads) {
    const int hq = idx / D;
    const int dim = idx % D;
    float M = sm_m[hq][0];
#pragma unroll
    for (int s = 1; s < NSTATE; ++s) M = fmaxf(M, sm_m[hq][s]);
    float a = 0.f, L = 0.f;
#pragma unroll
    for (int s = 0; s < NSTATE; ++s) {
      const float w = __builtin_amdgcn_exp2f(sm_m[hq][s] - M);
      a = fmaf(w, sm_acc[hq][s][dim], a);
      L = fmaf(w, sm_l[hq][s], L);
    }
    size_t slot;
    if constexpr (kRows<GR>) {  // the pair's position and head, recomputed (hq varies here)
      const int pi = hc * NQ + hq;
      const int gp = pi < n_pairs ? pos[pi / G] : -1;
      if (gp < 0 || gp >= W) continue;
      if (S == 1) {
        Elem<E>::store(out + ((size_t)(kvh * G + pi % G) * W + gp) * D + dim, L > 0.f ? a / L : 0.f);
        continue;
      }
      slot = ((size_t)kvh * n_pairs + pi) * S + split;
    } else if constexpr (GR == 3) {  // always a partial; one more slot per row
      slot = ((size_t)b * Hq + h0 + hq) * (S + 1) + split;
    } else if constexpr (GR == 4) {  // one split, sinks included: the output
      Elem<E>::store(out + ((size_t)b * Hq + h0 + hq) * D + dim, L > 0.f ? a / L : 0.f);
      continue;
    } else {
      if (S == 1) {  // no other split to merge with: finish here
        Elem<E>::store(out + ((size_t)b * Hq + h0 + hq) * D + dim, L > 0.f ? a / L : 0.f);
        continue;
      }
      slot = ((size_t)b * Hq + h0 + hq) * S + split;
    }
    ws_acc[slot * D + dim] = a;
    if (dim == 0) {
      ws_m[slot] = M;
      ws_l[slot] = L;
    }
  }
}

// ------------------------------------------------------------ attention sinks

// The sinks' partial of one (sequence, query head) for decode with sinks
// (Ultralytics glossary, terms section: StreamingLLM keeps the first tokens
// in the cache beside the window): the sink positions s < min(n_sink,
// p - W + 1), i.e. those before the window, read from k_sink / v_sink; the
// window's sinks are in the ring already.  One wave; written as partial S
// of the row's S + 1 (same units as the split pass: scores times
// scale * log2(e)).
template <typename E, int D>
__global__ __launch_bounds__(64) void sink_partial_kernel(
    const E* __restrict__ q, const E* __restrict__ k_sink, const E* __restrict__ v_sink,
    const int32_t* __restrict__ pos, float* __restrict__ ws_acc, float* __restrict__ ws_m,
    float* __restrict__ ws_l, int Hq, int Hkv, int W, int n_sink, float scale_log2, int S) {
  constexpr int DPL = (D + 63) / 64;  // dims per lane
  const size_t row = blockIdx.x;      // b * Hq + h
  const int b = (int)(row / Hq), h = (int)(row % Hq);
  const int kvh = h / (Hq / Hkv);
  const int lane = threadIdx.x;
  const int p = pos[b];
  const int ns = p < 0 ? 0 : min(n_sink, max(0, p - W + 1));
  float qv[DPL], acc[DPL];
#pragma unroll
  for (int j = 0; j < DPL; ++j) {
    const int dim = lane + 64 * j;
    qv[j] = dim < D ? static_cast<float>(q[row * D + dim]) : 0.f;
    acc[j] = 0.f;
  }
  float m = kNegBig, l = 0.f;
  const size_t base = ((size_t)b * Hkv + kvh) * (size_t)n_sink * D;
  for (int s = 0; s < ns; ++s) {
    float part = 0.f;
#pragma unroll
    for (int j = 0; j < DPL; ++j) {
      const int dim = lane + 64 * j;
      if (dim < D) part = fmaf(qv[j], static_cast<float>(k_sink[base + (size_t)s * D + dim]), part);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off);
    const float sc = part * scale_log2;
    const float m_new = fmaxf(m, sc);
    const float alpha = __builtin_amdgcn_exp2f(m - m_new);
    const float pr = __builtin_amdgcn_exp2f(sc - m_new);
    l = l * alpha + pr;
#pragma unroll
    for (int j = 0; j < DPL; ++j) {
      const int dim = lane + 64 * j;
      const float vv = dim < D ? static_cast<float>(v_sink[base + (size_t)s * D + dim]) : 0.f;
      acc[j] = fmaf(pr, vv, acc[j] * alpha);
    }
    m = m_new;
  }
  const size_t slot = row * (S + 1) + S;
#pragma unroll
  for (int j = 0; j < DPL; ++j) {
    const int dim = lane + 64 * j;
    if (dim < D) ws_acc[slot * D + dim] = acc[j];
  }
  if (lane == 0) {
    ws_m[slot] = m;
    ws_l[slot] = l;
  }
}

// ------------------------------------------------------------ split merge

template <typename E, int D, int GR>
__global__ __launch_bounds__(D) void decode_combine_kernel(const float* __restrict__ ws_acc,
                                                           const float* __restrict__ ws_m,
                                                           const float* __restrict__ ws_l,
                                                           E* __restrict__ out, int S,
                                                           const int32_t* __restrict__ gpos,
                                                           int T, int G, int n_pairs) {
  // b * Hq + h; GR != 0: kvh * n_pairs + pi for pair pi of KV head kvh
  const size_t row = blockIdx.x;
  const int dim = threadIdx.x;
  const float* m = ws_m + row * S;
  const float* l = ws_l + row * S;
  float M = m[0];
  float a = 0.f, L = 0.f;
  if constexpr (kRows<GR>) {  // many splits: several in flight at once
#pragma unroll kCombineUnroll
    for (int s = 1; s < S; ++s) M = fmaxf(M, m[s]);
#pragma unroll kCombineUnroll
    for (int s = 0; s < S; ++s) {
      const float w = __builtin_amdgcn_exp2f(m[s] - M);
      L = fmaf(w, l[s], L);
      a = fmaf(w, ws_acc[(row * S + s) * D + dim], a);
    }
  } else {
    for (int s = 1; s < S; ++s) M = fmaxf(M, m[s]);
    for (int s = 0; s < S; ++s) {
      const float w = __builtin_amdgcn_exp2f(m[s] - M);
      L = fmaf(w, l[s], L);
      a = fmaf(w, ws_acc[(row * S + s) * D + dim], a);
    }
  }
  size_t orow = row * D;
  if constexpr (kRows<GR>) {
    const int kvh = (int)(row / n_pairs), pi = (int)(row % n_pairs);
    const int p = gpos[pi / G];
    if (p < 0 || p >= T) return;
    orow = ((size_t)(kvh * G + pi % G) * T + p) * D;
  }
  Elem<E>::store(out + orow + dim, L > 0.f ? a / L : 0.f);
}

template <typename E, int D, int NQ, int GR>
hipError_t launch_decode_t(const void* q, const void* k_ring, const void* v_ring,
                           const int32_t* pos, void* out, int B, int Hq, int Hkv, int W,
                           float scale, float* workspace, hipStream_t stream,
                           const void* k_sink = nullptr, const void* v_sink = nullptr,
                           int n_sink = 0) {
  const int S = kRows<GR> ? global_splits(B, Hq, W) : decode_splits(B, Hq, W);
  const int chunk = (W + S - 1) / S;
  const int G = Hq / Hkv;
  // global rows: B (global rows) x G pairs per KV head, NQ per workgroup
  const int n_pairs = kRows<GR> ? B * G : 0;
  const int n_hchunks = kRows<GR> ? (n_pairs + NQ - 1) / NQ : G / NQ;
  const size_t rows = (size_t)B * Hq * (GR == 3 ? S + 1 : S);
  // a plain decode of one split writes the output itself: no workspace (it
  // may be null then)
  const bool partials = (GR != 0 && GR != 4) || S > 1;
  float* ws_acc = partials ? workspace : nullptr;
  float* ws_m = partials ? ws_acc + rows * D : nullptr;
  float* ws_l = partials ? ws_m + rows : nullptr;
  const long long nwg = (long long)(kRows<GR> ? 1 : B) * Hkv * n_hchunks * S;
  hipLaunchKernelGGL((decode_split_kernel<E, D, NQ, GR>), dim3((unsigned)nwg), dim3(kDecodeThreads), 0,
                     stream, static_cast<const E*>(q), static_cast<const E*>(k_ring),
                     static_cast<const E*>(v_ring), pos, static_cast<E*>(out), ws_acc, ws_m, ws_l,
                     Hq, Hkv, W, scale * kLog2e, S, chunk, n_hchunks, n_pairs,
                     static_cast<const E*>(k_sink), static_cast<const E*>(v_sink), n_sink);
  hipError_t e = hipGetLastError();
  if (GR == 3 || GR == 4) return e;  // GR 3: the sinks' partial and the merge follow
  if (e != hipSuccess || S == 1) return e;
  hipLaunchKernelGGL((decode_combine_kernel<E, D, GR>), dim3((unsigned)((size_t)B * Hq)), dim3(D), 0,
                     stream, ws_acc, ws_m, ws_l, static_cast<E*>(out), S, pos, W, G, n_pairs);
  return hipGetLastError();
}

template <typename E, int D, int GR>
hipError_t launch_decode_d(const void* q, const void* k_ring, const void* v_ring,
                           const int32_t* pos, void* out, int B, int Hq, int Hkv, int W,
                           float scale, float* workspace, hipStream_t stream) {
  const int G = Hq / Hkv;
  if constexpr (kRows<GR>)  // global rows: kGlobalNQ pairs per workgroup
    return launch_decode_t<E, D, kGlobalNQ, GR>(q, k_ring, v_ring, pos, out, B, Hq, Hkv, W, scale, workspace, stream);
  if (G % 4 == 0)
    return launch_decode_t<E, D, 4, GR>(q, k_ring, v_ring, pos, out, B, Hq, Hkv, W, scale, workspace, stream);
  if (G % 2 == 0)
    return launch_decode_t<E, D, 2, GR>(q, k_ring, v_ring, pos, out, B, Hq, Hkv, W, scale, workspace, stream);
  return launch_decode_t<E, D, 1, GR>(q, k_ring, v_ring, pos, out, B, Hq, Hkv, W, scale, workspace, stream);
}

template <typename E, int D>
hipError_t launch_decode_sinks_d(const void* q, const void* k_ring, const void* v_ring,
                                 const void* k_sink, const void* v_sink, int n_sink,
                                 const int32_t* pos, void* out, int B, int Hq, int Hkv, int W,
                                 float scale, float* workspace, hipStream_t stream) {
  const int G = Hq / Hkv;
  hipError_t e;
  if (decode_splits(B, Hq, W) == 1) {  // one split: the sinks join its online softmax
    if (G % 4 == 0)
      return launch_decode_t<E, D, 4, 4>(q, k_ring, v_ring, pos, out, B, Hq, Hkv, W, scale, nullptr, stream, k_sink, v_sink, n_sink);
    if (G % 2 == 0)
      return launch_decode_t<E, D, 2, 4>(q, k_ring, v_ring, pos, out, B, Hq, Hkv, W, scale, nullptr, stream, k_sink, v_sink, n_sink);
    return launch_decode_t<E, D, 1, 4>(q, k_ring, v_ring, pos, out, B, Hq, Hkv, W, scale, nullptr, stream, k_sink, v_sink, n_sink);
  }
  if (G % 4 == 0)
    e = launch_decode_t<E, D, 4, 3>(q, k_ring, v_ring, pos, out, B, Hq, Hkv, W, scale, workspace, stream);
  else if (G % 2 == 0)
    e = launch_decode_t<E, D, 2, 3>(q, k_ring, v_ring, pos, out, B, Hq, Hkv, W, scale, workspace, stream);
  else
    e = launch_decode_t<E, D, 1, 3>(q, k_ring, v_ring, pos, out, B, Hq, Hkv, W, scale, workspace, stream);
  if (e != hipSuccess) return e;
  const int S = decode_splits(B, Hq, W);
  const size_t rows = (size_t)B * Hq * (S + 1);
  float* ws_acc = workspace;
  float* ws_m = ws_acc + rows * D;
  float* ws_l = ws_m + rows;
  hipLaunchKernelGGL((sink_partial_kernel<E, D>), dim3((unsigned)((size_t)B * Hq)), dim3(64), 0,
                     stream, static_cast<const E*>(q), static_cast<const E*>(k_sink),
                     static_cast<const E*>(v_sink), pos, ws_acc, ws_m, ws_l, Hq, Hkv, W, n_sink,
                     scale * kLog2e, S);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<E, D, 0>), dim3((unsigned)((size_t)B * Hq)), dim3(D), 0,
                     stream, ws_acc, ws_m, ws_l, static_cast<E*>(out), S + 1,
                     static_cast<const int32_t*>(nullptr), 0, 1, 0);
  return hipGetLastError();
}

template <typename E, int GR>
hipError_t launch_decode_e(const void* q, const void* k_ring, const void* v_ring,
                           const int32_t* pos, void* out, int B, int Hq, int Hkv, int W, int d,
                           float scale, float* workspace, hipStream_t stream) {
  if (d == 32) return launch_decode_d<E, 32, GR>(q, k_ring, v_ring, pos, out, B, Hq, Hkv, W, scale, workspace, stream);
  if (d == 64) return launch_decode_d<E, 64, GR>(q, k_ring, v_ring, pos, out, B, Hq, Hkv, W, scale, workspace, stream);
  return launch_decode_d<E, 128, GR>(q, k_ring, v_ring, pos, out, B, Hq, Hkv, W, scale, workspace, stream);
}

}  // namespace

hipError_t launch_append(void* k_ring, void* v_ring, const int32_t* pos, const void* k_new,
                         const void* v_new, int B, int Hkv, int W, int row_bytes,
                         hipStream_t stream) {
  const int cpr = row_bytes / 16;
  const long long total = (long long)B * Hkv * cpr;
  const long long blocks = (total + 255) / 256;
  hipLaunchKernelGGL(append_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<uint4*>(k_ring), static_cast<uint4*>(v_ring), pos,
                     static_cast<const uint4*>(k_new), static_cast<const uint4*>(v_new), Hkv, W,
                     cpr, total);
  return hipGetLastError();
}

hipError_t launch_append_chunk(void* k_ring, void* v_ring, const int32_t* pos, const void* k,
                               const void* v, int B, int n, int Hkv, int W, int row_bytes,
                               hipStream_t stream) {
  int log_cpr = 0;  // row_bytes / 16 is a power of two (d in {32, 64, 128})
  while ((16 << log_cpr) < row_bytes) ++log_cpr;
  const int n0 = n > W ? n - W : 0;
  const long long total = ((long long)B * Hkv * (n - n0)) << log_cpr;  // < 2^31 (checked)
  const long long blocks = (total + 255) / 256;
  hipLaunchKernelGGL(append_chunk_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<uint4*>(k_ring), static_cast<uint4*>(v_ring), pos,
                     static_cast<const uint4*>(k), static_cast<const uint4*>(v), Hkv, n, n0, W,
                     log_cpr, (unsigned)total);
  return hipGetLastError();
}

int decode_splits(int B, int Hq, int W) {
  // Split each ring only as far as needed for ~kDecodeItems (sequence,
  // query head, split) items, enough work to fill the 256 CUs; a single
  // split needs no merge pass.  Never split below 64 slots.
  const long long heads = (long long)B * Hq;
  long long want = (kDecodeItems + heads - 1) / heads;
  if (want < 1) want = 1;
  const long long cap = (W + 63) / 64;
  return (int)(want < cap ? want : cap);
}

hipError_t launch_decode_sinks(const void* q, const void* k_ring, const void* v_ring,
                               const void* k_sink, const void* v_sink, int n_sink,
                               const int32_t* pos, void* out, int B, int Hq, int Hkv, int W,
                               int d, float scale, int dtype, float* workspace,
                               hipStream_t stream) {
  if (dtype == 1) {
    if (d == 32) return launch_decode_sinks_d<__bf16, 32>(q, k_ring, v_ring, k_sink, v_sink, n_sink, pos, out, B, Hq, Hkv, W, scale, workspace, stream);
    if (d == 64) return launch_decode_sinks_d<__bf16, 64>(q, k_ring, v_ring, k_sink, v_sink, n_sink, pos, out, B, Hq, Hkv, W, scale, workspace, stream);
    return launch_decode_sinks_d<__bf16, 128>(q, k_ring, v_ring, k_sink, v_sink, n_sink, pos, out, B, Hq, Hkv, W, scale, workspace, stream);
  }
  if (d == 32) return launch_decode_sinks_d<float, 32>(q, k_ring, v_ring, k_sink, v_sink, n_sink, pos, out, B, Hq, Hkv, W, scale, workspace, stream);
  if (d == 64) return launch_decode_sinks_d<float, 64>(q, k_ring, v_ring, k_sink, v_sink, n_sink, pos, out, B, Hq, Hkv, W, scale, workspace, stream);
  return launch_decode_sinks_d<float, 128>(q, k_ring, v_ring, k_sink, v_sink, n_sink, pos, out, B, Hq, Hkv, W, scale, workspace, stream);
}

hipError_t launch_global_combine(float* workspace, void* out, const int32_t* gpos, int ngl, int T,
                                 int Hq, int Hkv, int d, int S, int dtype, hipStream_t stream) {
  // merge of split partials laid out as the global-row pass writes them:
  // row kvh * n_pairs + pi, S partials each
  const size_t rows = (size_t)ngl * Hq;
  float* ws_acc = workspace;
  float* ws_m = ws_acc + rows * S * d;
  float* ws_l = ws_m + rows * S;
  const int G = Hq / Hkv;
  const int n_pairs = ngl * G;
#define SWA_COMBINE(E, DD)                                                                      \
  hipLaunchKernelGGL((decode_combine_kernel<E, DD, 1>), dim3((unsigned)rows), dim3(DD), 0, stream, \
                     ws_acc, ws_m, ws_l, static_cast<E*>(out), S, gpos, T, G, n_pairs)
  if (dtype == 1) {
    if (d == 32) SWA_COMBINE(__bf16, 32);
    else if (d == 64) SWA_COMBINE(__bf16, 64);
    else SWA_COMBINE(__bf16, 128);
  } else {
    if (d == 32) SWA_COMBINE(float, 32);
    else if (d == 64) SWA_COMBINE(float, 64);
    else SWA_COMBINE(float, 128);
  }
#undef SWA_COMBINE
  return hipGetLastError();
}

int global_splits(int G, int Hq, int T) {
  // ~kGlobalItems (row, head, split) items, never below 64 keys.  The
  // pass is bound by its vector arithmetic (one dot product, exponential
  // and d FMAs per key and pair), not by memory: finer splits (8192 items)
  // or 8 pairs per workgroup (registers for one wave per SIMD) measured
  // slower.  Its loads are ordinary (cached) ones: the windowed pass has just
  // read the same K/V.
  const long long rows = (long long)G * Hq;
  long long want = (kGlobalItems + rows - 1) / rows;
  if (want < 1) want = 1;
  const long long cap = (T + 63) / 64;
  return (int)(want < cap ? want : cap);
}

hipError_t launch_decode(const void* q, const void* k_ring, const void* v_ring,
                         const int32_t* pos, void* out, int B, int Hq, int Hkv, int W, int d,
                         float scale, int dtype, float* workspace, hipStream_t stream) {
  if (dtype == 1)
    return launch_decode_e<__bf16, 0>(q, k_ring, v_ring, pos, out, B, Hq, Hkv, W, d, scale, workspace, stream);
  return launch_decode_e<float, 0>(q, k_ring, v_ring, pos, out, B, Hq, Hkv, W, d, scale, workspace, stream);
}

hipError_t launch_global_rows_f32(const void* q, const void* k, const void* v, const int32_t* gpos,
                                  void* out, int ngl, int T, int Hq, int Hkv, int d, int mode,
                                  float scale, float* workspace, hipStream_t stream) {
  // ngl "sequences" (the global rows), each against the whole K/V as a ring of T slots
  if (mode == 0)
    return launch_decode_e<float, 1>(q, k, v, gpos, out, ngl, Hq, Hkv, T, d, scale, workspace, stream);
  return launch_decode_e<float, 2>(q, k, v, gpos, out, ngl, Hq, Hkv, T, d, scale, workspace, stream);
}

// ------------------------------------------------- library-owned scratch

// Split partials of swa_decode_noalloc, for callers that cannot allocate.
// One copy per GPU (each device holds its own instance of the array, at its
// own address) lives until the process ends.  Host code never passes the
// array's name to a kernel or a copy: in host code it is a stand-in, not a
// device address; the address comes from hipGetSymbolAddress, once per
// device, with that device current.
constexpr int kMaxScratchDevices = 64;
static __device__ __align__(256) float scratch[kDecodeScratchBytes / sizeof(float)];

namespace {
std::mutex g_scratch_mu;
float* g_scratch[kMaxScratchDevices];  // per device; null until first use
}  // namespace

hipError_t decode_scratch(hipStream_t stream, float** ptr) {
  int dev = 0;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    const hipError_t back = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return e;
    if (back != hipSuccess) return back;
    g_scratch[dev] = static_cast<float*>(p);
  }
  *ptr = g_scratch[dev];
  return hipSuccess;
}

}  // namespace swa
