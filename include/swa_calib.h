/*
 * swa_calib.h - calibration kernels shipped in the same library as swa.h.
 *
 * They compute nothing of the attention method.  They measure, on the GPU the
 * attention kernels run on, the two ceilings those kernels are bound by (the
 * matrix-core rate on random bf16 operands and the streaming HBM read rate),
 * so that the attention kernels' throughput can be quoted against what the
 * chip sustains as well as against its published peaks.  Status codes are the
 * swa_status values of swa.h.
 */
#ifndef SWA_CALIB_H
#define SWA_CALIB_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * swa_calib_mfma_bf16 - n_wg workgroups of four waves; each wave runs
 * iters x 16 v_mfma_f32_32x32x16_bf16 (32,768 FLOPs each) on operands taken
 * from `operands` (device, bf16 bits, operand_bytes a multiple of 16, at
 * least 16; random data gives the chip's power-limited rate, which is what
 * attention operands see), rotating four A and four B fragments per lane
 * over four accumulator chains.  Total FLOPs = n_wg * 4 * iters * 16 * 32768.
 *   sink   output float [n_wg * 256] (per-lane sums, keeps the work live).
 *   Errors: SWA_ERR_INVALID_ARG for null or unaligned pointers, bad sizes,
 *   n_wg outside [1, 2^20], iters < 0; SWA_ERR_LAUNCH on launch failure.
 *
 * swa_calib_stream_read - reads `bytes` (a multiple of 16) from device memory
 * `src` with 16-byte non-temporal loads: workgroup w of n_wg (256 lanes,
 * eight loads in flight per lane) reads the w-th contiguous chunk.  Use a
 * buffer larger than the 256 MB Infinity Cache to measure HBM.
 *   sink   output uint32 [n_wg * 256] (XOR of what each lane read).
 *   Errors as above (n_wg >= 1).
 *
 * Both are asynchronous on `stream`; time them with events on that stream.
 */
int swa_calib_mfma_bf16(const void* operands, size_t operand_bytes, float* sink, int n_wg,
                        int iters, void* stream);
int swa_calib_stream_read(const void* src, size_t bytes, unsigned* sink, int n_wg,
                          void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SWA_CALIB_H */
