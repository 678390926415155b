// C ABI of the SWA library: host-side argument checks, then dispatch to the
// gfx950 kernels.  The checks run before any HIP call, so an invalid call
// never touches the device (and can be exercised on a machine without one).

#include <math.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "swa.h"
#include "swa_calib.h"
#include "swa_launch.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool supported_d(int d) { return d == 32 || d == 64 || d == 128; }

bool known_dtype(int dtype) { return dtype == SWA_F32 || dtype == SWA_BF16; }

int elem_bytes(int dtype) { return dtype == SWA_BF16 ? 2 : 4; }

constexpr long long kMaxGrid = 2147483647LL;

// Longest sequence (and chunk) a prefill call takes: row and key indices, and
// the ends of a block's key range (row + 127 + W / 2 after the clamp below),
// stay inside int32.
constexpr int kMaxSeq = 1 << 29;

// |scale| above this is rejected.  The kernels form the softmax exponent
// scale * log2(e) * (s - m) as one fp32 fused multiply-add, s * c - m * c,
// whose rounding is about |s * c| * 2^-24: at |scale| <= 1024 it stays below
// 0.01 (a bf16-level error in the probability) for scores up to 100 in
// magnitude, and the starting reference -1e30 * c stays finite.  Attention
// scales are 1/sqrt(d) <= 1; a softmax at |scale| = 1024 is already a hard
// maximum for scores that differ by more than a few hundredths.
constexpr float kMaxScale = 1024.0f;

bool scale_ok(float scale) { return isfinite(scale) && fabsf(scale) <= kMaxScale; }

// A window wider than the sequence sees every key it can: W >= T (causal) and
// floor(W / 2) >= T - 1 (symmetric) are both full attention, also on a
// dilation grid, so W is clamped to 2T before launch (exact).
int clamp_window(int W, int T) { return (long long)W > 2LL * T ? 2 * T : W; }

}  // namespace

extern "C" {

int swa_prefill(const void* q, const void* k, const void* v, void* out, int T, int W, int Hq,
                int Hkv, int d, int mode, float scale, int dtype, void* stream) {
  if (!q || !k || !v || !out) return SWA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return SWA_ERR_INVALID_ARG;
  if (T <= 0 || W <= 0 || Hq <= 0 || Hkv <= 0) return SWA_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return SWA_ERR_INVALID_ARG;
  if (!scale_ok(scale)) return SWA_ERR_INVALID_ARG;
  if (!supported_d(d) || !known_dtype(dtype)) return SWA_ERR_UNSUPPORTED;
  if (mode != SWA_CAUSAL && mode != SWA_SYMMETRIC) return SWA_ERR_UNSUPPORTED;
  if (T > kMaxSeq) return SWA_ERR_UNSUPPORTED;
  // workgroup count must fit the grid (bounded with 16 rows per workgroup:
  // every kernel takes at least 32)
  if ((long long)((T + 15) / 16) * Hq > kMaxGrid) return SWA_ERR_UNSUPPORTED;
  W = clamp_window(W, T);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = (dtype == SWA_BF16)
                     ? swa::launch_prefill_bf16(q, k, v, out, T, W, Hq, Hkv, d, mode, scale, s)
                     : swa::launch_prefill_f32(q, k, v, out, T, W, Hq, Hkv, d, mode, scale, s);
  return e == hipSuccess ? SWA_OK : SWA_ERR_LAUNCH;
}

int swa_prefill_dilated(const void* q, const void* k, const void* v, void* out, int T, int W,
                        int Hq, int Hkv, int d, int mode, float scale, int dilation, int dtype,
                        void* stream) {
  if (!q || !k || !v || !out) return SWA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return SWA_ERR_INVALID_ARG;
  if (T <= 0 || W <= 0 || Hq <= 0 || Hkv <= 0 || dilation <= 0) return SWA_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return SWA_ERR_INVALID_ARG;
  if (!scale_ok(scale)) return SWA_ERR_INVALID_ARG;
  if (!supported_d(d) || !known_dtype(dtype)) return SWA_ERR_UNSUPPORTED;
  if (mode != SWA_CAUSAL && mode != SWA_SYMMETRIC) return SWA_ERR_UNSUPPORTED;
  if (T > kMaxSeq) return SWA_ERR_UNSUPPORTED;
  // a tile's 64 rows, dilation rows apart, are addressed with 32-bit byte offsets
  if ((long long)dilation * d * elem_bytes(dtype) * 64 > 2147483647LL) return SWA_ERR_UNSUPPORTED;
  // workgroup counts: at least 32 rows per workgroup (bounded with 16); 128-row
  // blocks of each residue class
  if ((long long)((T + 15) / 16) * Hq > kMaxGrid) return SWA_ERR_UNSUPPORTED;
  const long long class_rows = (T + (long long)dilation - 1) / dilation;
  if ((class_rows + 127) / 128 * Hq * (long long)dilation > kMaxGrid) return SWA_ERR_UNSUPPORTED;
  W = clamp_window(W, T);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e =
      (dtype == SWA_BF16)
          ? swa::launch_prefill_dilated_bf16(q, k, v, out, T, W, Hq, Hkv, d, mode, scale, dilation, s)
          : swa::launch_prefill_dilated_f32(q, k, v, out, T, W, Hq, Hkv, d, mode, scale, dilation, s);
  return e == hipSuccess ? SWA_OK : SWA_ERR_LAUNCH;
}

// Window (dilated when dilation > 1) plus global tokens: the window pass
// visits the global keys, then the global rows are computed over every key.
static int prefill_global_impl(const void* q, const void* k, const void* v, void* out, int T,
                               int W, int Hq, int Hkv, int d, int mode, float scale,
                               int dilation, const int32_t* global_pos, int G, void* workspace,
                               size_t workspace_bytes, int dtype, void* stream) {
  if (!q || !k || !v || !out || !global_pos) return SWA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(global_pos))
    return SWA_ERR_INVALID_ARG;
  if (T <= 0 || W <= 0 || Hq <= 0 || Hkv <= 0 || G < 0 || dilation <= 0) return SWA_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return SWA_ERR_INVALID_ARG;
  if (!scale_ok(scale)) return SWA_ERR_INVALID_ARG;
  if (!supported_d(d) || !known_dtype(dtype)) return SWA_ERR_UNSUPPORTED;
  if (mode != SWA_CAUSAL && mode != SWA_SYMMETRIC) return SWA_ERR_UNSUPPORTED;
  // global keys are gathered with 32-bit byte offsets into a head's K/V, and
  // a tile's 64 rows, dilation rows apart, likewise
  if ((long long)T * d * elem_bytes(dtype) > 2147483647LL) return SWA_ERR_UNSUPPORTED;
  if ((long long)dilation * d * elem_bytes(dtype) * 64 > 2147483647LL) return SWA_ERR_UNSUPPORTED;
  if ((long long)((T + 15) / 16) * Hq > kMaxGrid) return SWA_ERR_UNSUPPORTED;
  const long long class_rows = (T + (long long)dilation - 1) / dilation;
  if ((class_rows + 127) / 128 * Hq * (long long)dilation > kMaxGrid) return SWA_ERR_UNSUPPORTED;
  const int S = swa::global_splits(G, Hq, T);
  if ((long long)G * Hq * S > kMaxGrid) return SWA_ERR_UNSUPPORTED;
  const int S1 = swa::global_rows_mfma_splits(T);
  // bf16: the window workgroups and the global-row workgroups (two units
  // each) share one launch
  const long long row_units = (long long)Hkv * ((G * (Hq / Hkv) + 31) / 32) * S1;
  if ((class_rows + 127) / 128 * Hq * (long long)dilation + (row_units + 1) / 2 + 8 > kMaxGrid)
    return SWA_ERR_UNSUPPORTED;
  const size_t need = swa_prefill_global_workspace_bytes(T, Hq, G, d);
  if (!workspace || !aligned16(workspace) || workspace_bytes < need) return SWA_ERR_WORKSPACE;
  W = clamp_window(W, T);
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* ws = static_cast<float*>(workspace);
  hipError_t e = (dtype == SWA_BF16)
                     // the window pass and, in the same launch, the global rows'
                     // split-K partials on the matrix cores
                     ? swa::launch_prefill_global_window_bf16(q, k, v, out, T, W, Hq, Hkv, d, mode,
                                                              scale, global_pos, G, dilation, ws, s)
                     : swa::launch_prefill_global_window_f32(q, k, v, out, T, W, Hq, Hkv, d, mode,
                                                             scale, global_pos, G, dilation, s);
  if (e != hipSuccess) return SWA_ERR_LAUNCH;
  if (dtype == SWA_BF16) {  // the merge of the global rows' partials
    e = swa::launch_global_combine(ws, out, global_pos, G, T, Hq, Hkv, d,
                                   swa::global_rows_mfma_splits(T), dtype, s);
  } else {
    e = swa::launch_global_rows_f32(q, k, v, global_pos, out, G, T, Hq, Hkv, d, mode, scale, ws, s);
  }
  return e == hipSuccess ? SWA_OK : SWA_ERR_LAUNCH;
}

int swa_prefill_global(const void* q, const void* k, const void* v, void* out, int T, int W,
                       int Hq, int Hkv, int d, int mode, float scale, const int32_t* global_pos,
                       int G, void* workspace, size_t workspace_bytes, int dtype, void* stream) {
  if (G == 0)
    return swa_prefill(q, k, v, out, T, W, Hq, Hkv, d, mode, scale, dtype, stream);
  return prefill_global_impl(q, k, v, out, T, W, Hq, Hkv, d, mode, scale, 1, global_pos, G,
                             workspace, workspace_bytes, dtype, stream);
}

int swa_prefill_dilated_global(const void* q, const void* k, const void* v, void* out, int T,
                               int W, int Hq, int Hkv, int d, int mode, float scale, int dilation,
                               const int32_t* global_pos, int G, void* workspace,
                               size_t workspace_bytes, int dtype, void* stream) {
  if (G == 0)
    return swa_prefill_dilated(q, k, v, out, T, W, Hq, Hkv, d, mode, scale, dilation, dtype,
                               stream);
  if (dilation == 1)
    return swa_prefill_global(q, k, v, out, T, W, Hq, Hkv, d, mode, scale, global_pos, G,
                              workspace, workspace_bytes, dtype, stream);
  return prefill_global_impl(q, k, v, out, T, W, Hq, Hkv, d, mode, scale, dilation, global_pos, G,
                             workspace, workspace_bytes, dtype, stream);
}

int swa_cache_append(void* k_ring, void* v_ring, const int32_t* pos, const void* k_new,
                     const void* v_new, int B, int Hkv, int W, int d, int dtype, void* stream) {
  if (!k_ring || !v_ring || !pos || !k_new || !v_new) return SWA_ERR_INVALID_ARG;
  if (!aligned16(k_ring) || !aligned16(v_ring) || !aligned16(pos) || !aligned16(k_new) ||
      !aligned16(v_new))
    return SWA_ERR_INVALID_ARG;
  if (B <= 0 || Hkv <= 0 || W <= 0) return SWA_ERR_INVALID_ARG;
  if (!supported_d(d) || !known_dtype(dtype)) return SWA_ERR_UNSUPPORTED;
  const long long row_bytes = (long long)d * elem_bytes(dtype);
  if ((long long)B * Hkv * (row_bytes / 16) / 256 + 1 > kMaxGrid) return SWA_ERR_UNSUPPORTED;
  hipError_t e = swa::launch_append(k_ring, v_ring, pos, k_new, v_new, B, Hkv, W, (int)row_bytes,
                                    static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SWA_OK : SWA_ERR_LAUNCH;
}

int swa_cache_append_chunk(void* k_ring, void* v_ring, const int32_t* pos, const void* k,
                           const void* v, int B, int n, int Hkv, int W, int d, int dtype,
                           void* stream) {
  if (!k_ring || !v_ring || !pos || !k || !v) return SWA_ERR_INVALID_ARG;
  if (!aligned16(k_ring) || !aligned16(v_ring) || !aligned16(pos) || !aligned16(k) ||
      !aligned16(v))
    return SWA_ERR_INVALID_ARG;
  if (B <= 0 || n <= 0 || Hkv <= 0 || W <= 0) return SWA_ERR_INVALID_ARG;
  if (!supported_d(d) || !known_dtype(dtype)) return SWA_ERR_UNSUPPORTED;
  const long long row_bytes = (long long)d * elem_bytes(dtype);
  const long long written = n < W ? n : W;
  // one thread per 16 bytes written, indexed in 32 bits
  if ((long long)B * Hkv * written * (row_bytes / 16) > 2147483647LL) return SWA_ERR_UNSUPPORTED;
  hipError_t e = swa::launch_append_chunk(k_ring, v_ring, pos, k, v, B, n, Hkv, W, (int)row_bytes,
                                          static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SWA_OK : SWA_ERR_LAUNCH;
}

int swa_prefill_chunk(const void* q, const void* k, const void* v, const void* k_ring,
                      const void* v_ring, const int32_t* pos, void* out, int B, int n, int W,
                      int Hq, int Hkv, int d, float scale, int dtype, void* stream) {
  if (!q || !k || !v || !k_ring || !v_ring || !pos || !out) return SWA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(k_ring) ||
      !aligned16(v_ring) || !aligned16(pos) || !aligned16(out))
    return SWA_ERR_INVALID_ARG;
  if (B <= 0 || n <= 0 || W <= 0 || Hq <= 0 || Hkv <= 0) return SWA_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return SWA_ERR_INVALID_ARG;
  if (!scale_ok(scale)) return SWA_ERR_INVALID_ARG;
  if (!supported_d(d) || !known_dtype(dtype)) return SWA_ERR_UNSUPPORTED;
  if (n > kMaxSeq) return SWA_ERR_UNSUPPORTED;
  // ring rows are addressed with 32-bit byte offsets
  if ((long long)W * d * elem_bytes(dtype) > 2147483647LL) return SWA_ERR_UNSUPPORTED;
  // folded head counts and the workgroup count (bounded with 16 rows per
  // workgroup) fit int32
  if ((long long)B * Hq > kMaxGrid) return SWA_ERR_UNSUPPORTED;
  if ((long long)((n + 15) / 16) * Hq * B > kMaxGrid) return SWA_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e =
      (dtype == SWA_BF16)
          ? swa::launch_prefill_chunk_bf16(q, k, v, k_ring, v_ring, pos, out, B, n, W, Hq, Hkv, d,
                                           scale, s)
          : swa::launch_prefill_chunk_f32(q, k, v, k_ring, v_ring, pos, out, B, n, W, Hq, Hkv, d,
                                          scale, s);
  return e == hipSuccess ? SWA_OK : SWA_ERR_LAUNCH;
}

size_t swa_prefill_global_workspace_bytes(int T, int Hq, int G, int d) {
  if (T <= 0 || Hq <= 0 || G <= 0 || !supported_d(d)) return 0;
  // the larger of the two global-row passes (matrix cores for bf16, vector
  // units for fp32)
  const int S0 = swa::global_splits(G, Hq, T);
  const int S1 = swa::global_rows_mfma_splits(T);
  return (size_t)G * Hq * (S0 > S1 ? S0 : S1) * (size_t)(d + 2) * sizeof(float);
}

size_t swa_decode_workspace_bytes(int B, int Hq, int W, int d) {
  if (B <= 0 || Hq <= 0 || W <= 0 || !supported_d(d)) return 0;
  const int S = swa::decode_splits(B, Hq, W);
  if (S == 1) return 0;  // one split writes the output itself: no partials
  return (size_t)B * Hq * S * (size_t)(d + 2) * sizeof(float);
}

int swa_decode(const void* q, const void* k_ring, const void* v_ring, const int32_t* pos,
               void* out, int B, int Hq, int Hkv, int W, int d, float scale, int dtype,
               void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k_ring || !v_ring || !pos || !out) return SWA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_ring) || !aligned16(v_ring) || !aligned16(pos) ||
      !aligned16(out))
    return SWA_ERR_INVALID_ARG;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || W <= 0) return SWA_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return SWA_ERR_INVALID_ARG;
  if (!scale_ok(scale)) return SWA_ERR_INVALID_ARG;
  if (!supported_d(d) || !known_dtype(dtype)) return SWA_ERR_UNSUPPORTED;
  const size_t need = swa_decode_workspace_bytes(B, Hq, W, d);
  if (need > 0 && (!workspace || !aligned16(workspace) || workspace_bytes < need))
    return SWA_ERR_WORKSPACE;
  const int S = swa::decode_splits(B, Hq, W);
  if ((long long)B * Hq * S > kMaxGrid) return SWA_ERR_UNSUPPORTED;
  hipError_t e = swa::launch_decode(q, k_ring, v_ring, pos, out, B, Hq, Hkv, W, d, scale, dtype,
                                    static_cast<float*>(workspace),
                                    static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SWA_OK : SWA_ERR_LAUNCH;
}

int swa_decode_noalloc(const void* q, const void* k_ring, const void* v_ring, const int32_t* pos,
                       void* out, int B, int Hq, int Hkv, int W, int d, float scale, int dtype,
                       void* stream) {
  if (!q || !k_ring || !v_ring || !pos || !out) return SWA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_ring) || !aligned16(v_ring) || !aligned16(pos) ||
      !aligned16(out))
    return SWA_ERR_INVALID_ARG;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || W <= 0) return SWA_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return SWA_ERR_INVALID_ARG;
  if (!scale_ok(scale)) return SWA_ERR_INVALID_ARG;
  if (!supported_d(d) || !known_dtype(dtype)) return SWA_ERR_UNSUPPORTED;
  const size_t need = swa_decode_workspace_bytes(B, Hq, W, d);
  if (need > swa::kDecodeScratchBytes) return SWA_ERR_UNSUPPORTED;
  const int S = swa::decode_splits(B, Hq, W);
  if ((long long)B * Hq * S > kMaxGrid) return SWA_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* ws = nullptr;
  if (need > 0 && swa::decode_scratch(s, &ws) != hipSuccess) return SWA_ERR_LAUNCH;
  hipError_t e = swa::launch_decode(q, k_ring, v_ring, pos, out, B, Hq, Hkv, W, d, scale, dtype,
                                    ws, s);
  return e == hipSuccess ? SWA_OK : SWA_ERR_LAUNCH;
}

size_t swa_decode_sinks_workspace_bytes(int B, int Hq, int W, int d) {
  if (B <= 0 || Hq <= 0 || W <= 0 || !supported_d(d)) return 0;
  const int S = swa::decode_splits(B, Hq, W);
  return (size_t)B * Hq * (S + 1) * (size_t)(d + 2) * sizeof(float);
}

int swa_decode_sinks(const void* q, const void* k_ring, const void* v_ring, const void* k_sink,
                     const void* v_sink, int n_sink, const int32_t* pos, void* out, int B, int Hq,
                     int Hkv, int W, int d, float scale, int dtype, void* workspace,
                     size_t workspace_bytes, void* stream) {
  if (n_sink == 0)
    return swa_decode(q, k_ring, v_ring, pos, out, B, Hq, Hkv, W, d, scale, dtype, workspace,
                      workspace_bytes, stream);
  if (!q || !k_ring || !v_ring || !k_sink || !v_sink || !pos || !out) return SWA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_ring) || !aligned16(v_ring) || !aligned16(k_sink) ||
      !aligned16(v_sink) || !aligned16(pos) || !aligned16(out))
    return SWA_ERR_INVALID_ARG;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || W <= 0 || n_sink < 0) return SWA_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return SWA_ERR_INVALID_ARG;
  if (!scale_ok(scale)) return SWA_ERR_INVALID_ARG;
  if (!supported_d(d) || !known_dtype(dtype)) return SWA_ERR_UNSUPPORTED;
  const size_t need = swa_decode_sinks_workspace_bytes(B, Hq, W, d);
  if (!workspace || !aligned16(workspace) || workspace_bytes < need) return SWA_ERR_WORKSPACE;
  const int S = swa::decode_splits(B, Hq, W);
  if ((long long)B * Hq * (S + 1) > kMaxGrid) return SWA_ERR_UNSUPPORTED;
  hipError_t e = swa::launch_decode_sinks(q, k_ring, v_ring, k_sink, v_sink, n_sink, pos, out, B,
                                          Hq, Hkv, W, d, scale, dtype,
                                          static_cast<float*>(workspace),
                                          static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SWA_OK : SWA_ERR_LAUNCH;
}

int swa_calib_mfma_bf16(const void* operands, size_t operand_bytes, float* sink, int n_wg,
                        int iters, void* stream) {
  if (!operands || !sink) return SWA_ERR_INVALID_ARG;
  if (!aligned16(operands) || !aligned16(sink)) return SWA_ERR_INVALID_ARG;
  if (operand_bytes < 16 || operand_bytes % 16 != 0) return SWA_ERR_INVALID_ARG;
  if (operand_bytes / 16 > 2147483647ULL) return SWA_ERR_UNSUPPORTED;
  // fragment indices 8 * (workgroup * 256 + lane) + 7 stay in int
  if (n_wg <= 0 || n_wg > (1 << 20) || iters < 0) return SWA_ERR_INVALID_ARG;
  const hipError_t e = swa::launch_calib_mfma(operands, (int)(operand_bytes / 16), sink, n_wg,
                                              iters, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SWA_OK : SWA_ERR_LAUNCH;
}

int swa_calib_stream_read(const void* src, size_t bytes, unsigned* sink, int n_wg,
                          void* stream) {
  if (!src || !sink) return SWA_ERR_INVALID_ARG;
  if (!aligned16(src) || !aligned16(sink)) return SWA_ERR_INVALID_ARG;
  if (bytes < 16 || bytes % 16 != 0 || n_wg <= 0) return SWA_ERR_INVALID_ARG;
  if ((long long)n_wg > kMaxGrid / 256) return SWA_ERR_UNSUPPORTED;
  const hipError_t e =
      swa::launch_calib_read(src, bytes / 16, sink, n_wg, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SWA_OK : SWA_ERR_LAUNCH;
}

int swa_calib_vector(int op, float* sink, int n_wg, int iters, void* stream) {
  if (op != 0 && op != 1) return SWA_ERR_INVALID_ARG;
  if (!sink || !aligned16(sink)) return SWA_ERR_INVALID_ARG;
  if (n_wg <= 0 || n_wg > (1 << 20) || iters < 0) return SWA_ERR_INVALID_ARG;
  const hipError_t e =
      swa::launch_calib_vector(op, sink, n_wg, iters, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SWA_OK : SWA_ERR_LAUNCH;
}

const char* swa_status_string(int status) {
  switch (status) {
    case SWA_OK:
      return "ok";
    case SWA_ERR_INVALID_ARG:
      return "invalid argument";
    case SWA_ERR_UNSUPPORTED:
      return "unsupported configuration";
    case SWA_ERR_WORKSPACE:
      return "workspace missing or too small";
    case SWA_ERR_LAUNCH:
      return "kernel launch failed";
    default:
      return "unknown status";
  }
}

}  // extern "C"
