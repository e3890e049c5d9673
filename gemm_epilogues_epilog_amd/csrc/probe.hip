// MFMA issue-rate probe: back-to-back v_mfma_f32_32x32x16_{f16,bf16} on operand values
// the caller supplies, with nothing else in the loop (no memory traffic, no LDS).
// It measures what the matrix cores sustain on given data under the chip's power
// limit: the clock, and so the rate, depends on the operand values (random values
// toggle far more multiplier bits than constant ones). The fused kernels' fraction of
// the dense fp16/bf16 peak is read against it. Declared in include/gemm_epilog_probe.h.
#include <hip/hip_runtime.h>

#include "gemm_epilog_probe.h"
#include "kernels.hpp"

namespace gek {

constexpr int kProbeThreads = 256;   // four waves, one per SIMD
constexpr int kProbeChains = 4;      // independent accumulators per wave

// Each lane takes four 16-byte operand registers from `ops` (nops entries, wrapping):
// two operand pairs that consecutive MFMAs alternate between, so the multiplier inputs
// change from one MFMA to the next as they do in a GEMM. It issues kProbeChains MFMAs
// per iteration into independent accumulators; the sum of its accumulators goes to
// out[global thread], so nothing is dead code.
template <int DT>
__global__ __launch_bounds__(kProbeThreads) void mfma_probe_kernel(const i32x4* __restrict__ ops, int nops,
                                                                   int iters, float* __restrict__ out) {
  const int t = blockIdx.x * kProbeThreads + threadIdx.x;
  const i32x4 a0 = ops[t % nops];
  const i32x4 b0 = ops[(t + 1) % nops];
  const i32x4 a1 = ops[(t + 2) % nops];
  const i32x4 b1 = ops[(t + 3) % nops];
  f32x16 acc[kProbeChains];
#pragma unroll
  for (int j = 0; j < kProbeChains; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kProbeChains; ++j) acc[j] = (j & 1) ? Tr<DT>::mma(a1, b1, acc[j]) : Tr<DT>::mma(a0, b0, acc[j]);
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < kProbeChains; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  out[t] = s;
}

}  // namespace gek

extern "C" ge_status_t gemm_epilog_mfma_probe(const void* operands, size_t operand_bytes, ge_dtype_t dt, int iters,
                                              int workgroups, float* out, void* stream) {
  if (!operands || !out) return GE_ERR_NULL_POINTER;
  if (dt != GE_F16 && dt != GE_BF16) return GE_ERR_NOT_SUPPORTED;
  if (operand_bytes < 16 || operand_bytes / 16 > 0x7fffffff || iters < 1 || workgroups < 1 ||
      workgroups > (1 << 20))
    return GE_ERR_INVALID_VALUE;
  if ((reinterpret_cast<uintptr_t>(operands) % 16) != 0 || (reinterpret_cast<uintptr_t>(out) % 4) != 0)
    return GE_ERR_MISALIGNED;
  const gek::i32x4* ops = static_cast<const gek::i32x4*>(operands);
  int nops = (int)(operand_bytes / 16);
  void* params[] = {&ops, &nops, &iters, &out};
  const void* fn = dt == GE_F16 ? reinterpret_cast<const void*>(&gek::mfma_probe_kernel<gek::F16>)
                                : reinterpret_cast<const void*>(&gek::mfma_probe_kernel<gek::BF16>);
  return hipLaunchKernel(fn, dim3(workgroups), dim3(gek::kProbeThreads), params, 0,
                         static_cast<hipStream_t>(stream)) == hipSuccess
             ? GE_OK
             : GE_ERR_HIP;
}

extern "C" ge_status_t gemm_epilog_device_info(int* compute_units, int* clock_khz) {
  if (!compute_units || !clock_khz) return GE_ERR_NULL_POINTER;
  int dev = 0, cus = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipDeviceGetAttribute(&khz, hipDeviceAttributeClockRate, dev) != hipSuccess)
    return GE_ERR_HIP;
  *compute_units = cus;
  *clock_khz = khz;
  return GE_OK;
}
