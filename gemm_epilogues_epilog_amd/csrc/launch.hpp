// Kernel-configuration table shared by the host runtime and the per-type
// instantiation units.
#pragma once

#include <hip/hip_runtime.h>

#include "gemm_dtl.hpp"
#include "gemm_generic.hpp"

namespace gek {

// Workgroup tile (BM x BN) and wave tile (WM x WN) of each configuration.
struct TileCfg {
  int bm, bn, wm, wn;
  const char* name;
};

enum CfgId { CFG_S = 0, CFG_M = 1, CFG_L = 2, CFG_COUNT = 3 };

constexpr TileCfg kTiles[CFG_COUNT] = {
    {64, 64, 32, 32, "S"},
    {128, 128, 64, 64, "M"},
    {256, 256, 128, 64, "L"},
};

inline int threads_of(const TileCfg& c) { return (c.bm / c.wm) * (c.bn / c.wn) * 64; }

using LaunchFn = hipError_t (*)(const Args&, int grid, hipStream_t);

// 16-bit types with tiles of at least 128 columns use the direct-to-LDS kernel;
// fp32 and the small tile use the register-staged kernel.
template <int DT, int EP, int BM, int BN, int WM, int WN>
hipError_t launch_gemm(const Args& a, int grid, hipStream_t s) {
  Args copy = a;
  void* params[] = {&copy};
  const void* fn;
  if constexpr (DT != F32 && BN >= 128)
    fn = reinterpret_cast<const void*>(&gemm_dtl_kernel<DT, EP, BM, BN, WM, WN>);
  else
    fn = reinterpret_cast<const void*>(&gemm_epilog_kernel<DT, EP, BM, BN, WM, WN>);
  return hipLaunchKernel(fn, dim3(grid), dim3((BM / WM) * (BN / WN) * 64), params, 0, s);
}

template <int DT, int EP>
LaunchFn pick_cfg(int cfg) {
  switch (cfg) {
    case CFG_S: return &launch_gemm<DT, EP, 64, 64, 32, 32>;
    case CFG_M: return &launch_gemm<DT, EP, 128, 128, 64, 64>;
    case CFG_L:
      if constexpr (DT != F32) return &launch_gemm<DT, EP, 256, 256, 128, 64>;
      return nullptr;
    default: return nullptr;
  }
}

template <int DT>
LaunchFn pick(int ep, int cfg) {
  switch (ep) {
    case NONE: return pick_cfg<DT, NONE>(cfg);
    case RELU_BIAS: return pick_cfg<DT, RELU_BIAS>(cfg);
    case GELU_BIAS: return pick_cfg<DT, GELU_BIAS>(cfg);
    case RELU_AUX_BIAS: return pick_cfg<DT, RELU_AUX_BIAS>(cfg);
    case DRELU_BGRAD: return pick_cfg<DT, DRELU_BGRAD>(cfg);
    case BIAS: return pick_cfg<DT, BIAS>(cfg);
    default: return nullptr;
  }
}

// Defined one per storage type, each in its own translation unit.
LaunchFn get_launch_f32(int ep, int cfg);
LaunchFn get_launch_f16(int ep, int cfg);
LaunchFn get_launch_bf16(int ep, int cfg);

// Elementwise kernels of the unfused chain and the bgrad second pass.
hipError_t launch_bias_add(int dt, const void* in, const void* bias, int vec_dt, void* out, int64_t m, int n,
                           hipStream_t s);
hipError_t launch_relu(int dt, const void* in, void* out, int64_t m, int n, hipStream_t s);
hipError_t launch_bgrad_reduce(const float* partial, int t, int64_t m, void* bgrad, int vec_dt, hipStream_t s);

}  // namespace gek
