/*
 * swa_calib.h - calibration kernels shipped in the same library as swa.h.
 *
 * They compute nothing of the attention method.  They measure, on the GPU the
 * attention kernels run on, the ceilings those kernels are bound by (the
 * matrix-core rate on random bf16 operands, the streaming HBM read rate, and
 * the vector ALU's issue rate of the softmax's FMAs and exponentials), so that
 * the attention kernels' throughput can be quoted against what the chip
 * sustains as well as against its published peaks.  Status codes are the
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
 * swa_calib_vector - n_wg workgroups of four waves; every lane runs sixteen
 * independent chains of `iters` steps of one vector operation: op 0 an fp32
 * FMA (x = fma(x, 0.999, 0.001)), op 1 a base-2 exponential on v_exp_f32
 * (x = -exp2(x)).  Wave instructions issued = n_wg * 4 * iters * 16.
 *   sink   output float [n_wg * 256] (per-lane sums, keeps the work live).
 *   Errors: SWA_ERR_INVALID_ARG for op outside {0, 1}, a null or unaligned
 *   sink, n_wg outside [1, 2^20], iters < 0; SWA_ERR_LAUNCH on launch failure.
 *
 * All three are asynchronous on `stream`; time them with events on that
 * stream.
 */
int swa_calib_mfma_bf16(const void* operands, size_t operand_bytes, float* sink, int n_wg,
                        int iters, void* stream);
int swa_calib_stream_read(const void* src, size_t bytes, unsigned* sink, int n_wg,
                          void* stream);
int swa_calib_vector(int op, float* sink, int n_wg, int iters, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SWA_CALIB_H */
