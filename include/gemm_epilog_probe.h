/*
 * gemm_epilog_probe.h - measurement aid for the fused GEMM + epilogue library (gfx950):
 * the rate the matrix cores sustain on given operand values.
 *
 * Not part of the epilogue path: exported by its own library, libgemm_epilog_probe.so,
 * which only the benchmark and its tests load. The fused kernels report their throughput as a
 * fraction of the dense fp16/bf16 MFMA peak (256 compute units x 2.4 GHz x 4096 flop
 * per clock). Under the power limit the clock, and so the reachable rate, depends on
 * the operand values. This probe issues nothing but MFMAs on the values it is given,
 * so its rate on the workloads' own value distribution is the practical ceiling for
 * any kernel on those values.
 */
#ifndef GEMM_EPILOG_PROBE_H_
#define GEMM_EPILOG_PROBE_H_

#include <stddef.h>

#include "gemm_epilog.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * gemm_epilog_mfma_probe - enqueue one probe kernel on `stream` and return.
 *   operands      : device, operand_bytes bytes of fp16 or bf16 values (16-byte aligned,
 *                   at least 16 bytes); thread t of the grid takes the 16-byte groups
 *                   t, t + 1 and t + 2, t + 3 (modulo the group count) as two operand
 *                   pairs, and consecutive MFMAs alternate between the pairs.
 *   dt            : GE_F16 or GE_BF16 (else GE_ERR_NOT_SUPPORTED).
 *   iters         : >= 1; each wave issues 4 * iters v_mfma_f32_32x32x16 (32768 flop each).
 *   workgroups    : 1 .. 2^20 workgroups of 256 threads (4 waves).
 *   out           : device, workgroups * 256 floats, written (a sum of each thread's
 *                   accumulators, kept so the work is not optimised away).
 *   stream        : a hipStream_t; NULL means the null stream.
 * Flop per launch: workgroups * 4 * 4 * iters * 32768. Returns GE_ERR_NULL_POINTER,
 * GE_ERR_INVALID_VALUE or GE_ERR_MISALIGNED before any HIP call, GE_ERR_HIP if the launch
 * fails. The caller synchronises and times (e.g. with HIP events around the launch).
 */
ge_status_t gemm_epilog_mfma_probe(const void* operands, size_t operand_bytes, ge_dtype_t dt, int iters,
                                   int workgroups, float* out, void* stream);

/*
 * gemm_epilog_device_info - what the current HIP device reports, for stating the peak
 * the measurements are read against: its compute units and its peak shader clock (kHz;
 * the clock the dense MFMA peak assumes, not the clock under load).
 *   compute_units, clock_khz : host pointers, written on success.
 * Returns GE_ERR_NULL_POINTER for a NULL pointer, GE_ERR_HIP if the runtime cannot answer.
 */
ge_status_t gemm_epilog_device_info(int* compute_units, int* clock_khz);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_EPILOG_PROBE_H_ */
