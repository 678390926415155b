// Internal launchers behind the C ABI (not exported).  Each one enqueues its
// kernels on `stream` and returns the launch status; arguments have already
// been validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace swa {

hipError_t launch_prefill_bf16(const void* q, const void* k, const void* v, void* out, int T,
                               int W, int Hq, int Hkv, int d, int mode, float scale,
                               hipStream_t stream);

hipError_t launch_prefill_f32(const void* q, const void* k, const void* v, void* out, int T,
                              int W, int Hq, int Hkv, int d, int mode, float scale,
                              hipStream_t stream);

// Dilated window (dilation dil >= 1; dil = 1 is swa_prefill's window).
hipError_t launch_prefill_dilated_bf16(const void* q, const void* k, const void* v, void* out,
                                       int T, int W, int Hq, int Hkv, int d, int mode,
                                       float scale, int dil, hipStream_t stream);

hipError_t launch_prefill_dilated_f32(const void* q, const void* k, const void* v, void* out,
                                      int T, int W, int Hq, int Hkv, int d, int mode, float scale,
                                      int dil, hipStream_t stream);

// Window (dilated when dil > 1) plus global keys for every row (the global
// rows are left for the global-row pass).
hipError_t launch_prefill_global_window_bf16(const void* q, const void* k, const void* v,
                                             void* out, int T, int W, int Hq, int Hkv, int d,
                                             int mode, float scale, const int32_t* gpos, int ngl,
                                             int dil, float* workspace, hipStream_t stream);

hipError_t launch_prefill_global_window_f32(const void* q, const void* k, const void* v,
                                            void* out, int T, int W, int Hq, int Hkv, int d,
                                            int mode, float scale, const int32_t* gpos, int ngl,
                                            int dil, hipStream_t stream);

// Decode with n_sink attention-sink slots beside the ring.  Workspace:
// B * Hq * (decode_splits(B, Hq, W) + 1) partial records of d + 2 floats.
hipError_t launch_decode_sinks(const void* q, const void* k_ring, const void* v_ring,
                               const void* k_sink, const void* v_sink, int n_sink,
                               const int32_t* pos, void* out, int B, int Hq, int Hkv, int W,
                               int d, float scale, int dtype, float* workspace,
                               hipStream_t stream);

// The rows of the global tokens on the matrix cores (bf16) are split-K
// partials of global_rows_mfma_splits(T) chunks, written to the workspace by
// launch_prefill_global_window_bf16 and merged by launch_global_combine.
int global_rows_mfma_splits(int T);
hipError_t launch_global_combine(float* workspace, void* out, const int32_t* gpos, int ngl, int T,
                                 int Hq, int Hkv, int d, int S, int dtype, hipStream_t stream);

// Number of key chunks the fp32 global-row pass splits each row into.
int global_splits(int G, int Hq, int T);

// The rows of the global tokens in fp32: each attends to every key (every
// earlier key when causal).  Workspace: G * Hq * global_splits(G, Hq, T)
// partial records of d + 2 floats.
hipError_t launch_global_rows_f32(const void* q, const void* k, const void* v, const int32_t* gpos,
                                  void* out, int ngl, int T, int Hq, int Hkv, int d, int mode,
                                  float scale, float* workspace, hipStream_t stream);

// Chunk of n tokens per sequence against its ring plus itself (causal).
hipError_t launch_prefill_chunk_bf16(const void* q, const void* k, const void* v,
                                     const void* k_ring, const void* v_ring, const int32_t* pos,
                                     void* out, int B, int n, int W, int Hq, int Hkv, int d,
                                     float scale, hipStream_t stream);

hipError_t launch_prefill_chunk_f32(const void* q, const void* k, const void* v,
                                    const void* k_ring, const void* v_ring, const int32_t* pos,
                                    void* out, int B, int n, int W, int Hq, int Hkv, int d,
                                    float scale, hipStream_t stream);

hipError_t launch_append_chunk(void* k_ring, void* v_ring, const int32_t* pos, const void* k,
                               const void* v, int B, int n, int Hkv, int W, int row_bytes,
                               hipStream_t stream);

hipError_t launch_append(void* k_ring, void* v_ring, const int32_t* pos, const void* k_new,
                         const void* v_new, int B, int Hkv, int W, int row_bytes,
                         hipStream_t stream);

// Number of slot chunks ("splits") the decode pass divides each ring into.
int decode_splits(int B, int Hq, int W);

// Size of the library-owned decode scratch (one per GPU): the split partials
// of any swa_decode call fit (B*Hq*splits < 4096 records of d + 2 <= 130
// floats whenever the ring is split at all).
constexpr size_t kDecodeScratchBytes = (size_t)4 << 20;

// Device address of the calling device's scratch (the device of `stream`,
// or the current one for the null stream), looked up on first use.
hipError_t decode_scratch(hipStream_t stream, float** ptr);

hipError_t launch_decode(const void* q, const void* k_ring, const void* v_ring,
                         const int32_t* pos, void* out, int B, int Hq, int Hkv, int W, int d,
                         float scale, int dtype, float* workspace, hipStream_t stream);

// Calibration: a matrix-core loop on random bf16 operands (nfrag 16-byte
// fragments), a streaming non-temporal read of n16 16-byte vectors, and
// vector-ALU chains (op 0 fp32 FMA, op 1 exp2).
hipError_t launch_calib_mfma(const void* ops, int nfrag, float* sink, int n_wg, int iters,
                             hipStream_t stream);
hipError_t launch_calib_read(const void* src, size_t n16, unsigned* sink, int n_wg,
                             hipStream_t stream);
hipError_t launch_calib_vector(int op, float* sink, int n_wg, int iters, hipStream_t stream);

}  // namespace swa
