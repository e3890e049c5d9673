// Kernel launchers of each tile configuration (tiles.hpp), shared by the host runtime
// and the per-type instantiation units.
#pragma once

#include <hip/hip_runtime.h>

#include "gemm_dtl.hpp"
#include "gemm_generic.hpp"
#include "tiles.hpp"

namespace gek {

using LaunchFn = hipError_t (*)(const Args&, int grid, hipStream_t);

template <int DT, int EP, int BM, int BN, int WM, int WN>
hipError_t launch_generic(const Args& a, int grid, hipStream_t s) {
  Args copy = a;
  void* params[] = {&copy};
  const void* fn = reinterpret_cast<const void*>(&gemm_epilog_kernel<DT, EP, BM, BN, WM, WN>);
  return hipLaunchKernel(fn, dim3(grid), dim3((BM / WM) * (BN / WN) * 64), params, 0, s);
}

// Main loop of a configuration: plain lockstep (every wave copies), lockstep with copies
// on half the waves, or the persistent kernel (interleaved reads, copies on half the
// waves; one workgroup per tile with the same loop where the persistent kernel does not
// apply).
enum Loop { LOCKSTEP = 0, LOCKSTEP_HALF = 1, PERSIST = 2 };

// MFMAs of a k-tile's last step that the persistent loop issues before its barrier
// (half of a k-step's MFMAs for waves with fewer than eight).
constexpr int kPersistPre = 4;
constexpr int persist_pre(int nmma) { return kPersistPre < nmma ? kPersistPre : nmma / 2; }

// LAY != 0 (an operand stored transposed): one workgroup per tile, plain lockstep loop.
template <int DT, int EP, int BM, int BN, int WM, int WN, int BK, int ST, int LOOP, int LAY = 0>
hipError_t launch_dtl(const Args& a, int grid, hipStream_t s) {
  Args copy = a;
  void* params[] = {&copy};
  const void* fn;
  constexpr bool ILV = LOOP == PERSIST;
  constexpr int CW = (LOOP == LOCKSTEP_HALF || LOOP == PERSIST) ? (BM / WM) * (BN / WN) / 2 : 0;
  if constexpr (LAY != 0) {
    static_assert(LOOP == LOCKSTEP || LOOP == LOCKSTEP_HALF || LOOP == PERSIST,
                  "transposed operands: plain lockstep loop or the persistent kernel");
    fn = reinterpret_cast<const void*>(&gemm_dtl_kernel<DT, EP, BM, BN, WM, WN, BK, ST, false, CW, LAY>);
    if constexpr (LOOP == PERSIST) {
      if (a.persist_grid > 0) {
        fn = reinterpret_cast<const void*>(
            &gemm_persist_kernel<DT, EP, BM, BN, WM, WN, BK, ST, CW, persist_pre((WM / 32) * (WN / 32)), LAY>);
        grid = a.persist_grid;
      }
    }
  } else {
    fn = reinterpret_cast<const void*>(&gemm_dtl_kernel<DT, EP, BM, BN, WM, WN, BK, ST, ILV, CW>);
    if constexpr ((BM / WM) * (BN / WN) == 8) {   // the split tail exists for the 8-wave tiles
      if (a.dp_tiles < grid) {
        fn = reinterpret_cast<const void*>(&gemm_sk_kernel<DT, EP, BM, BN, WM, WN, BK, ST, ILV, CW>);
        grid = a.dp_tiles + a.sk_wgs;
      }
    }
    if constexpr (LOOP == PERSIST) {
      if (a.dp_tiles == grid && a.persist_grid > 0) {
        fn = reinterpret_cast<const void*>(
            &gemm_persist_kernel<DT, EP, BM, BN, WM, WN, BK, ST, CW, persist_pre((WM / 32) * (WN / 32))>);
        grid = a.persist_grid;
      }
    }
  }
  return hipLaunchKernel(fn, dim3(grid), dim3((BM / WM) * (BN / WN) * 64), params, 0, s);
}

template <int DT, int EP>
LaunchFn pick_cfg(int cfg) {
  switch (cfg) {
    case CFG_S: return &launch_generic<DT, EP, 64, 64, 32, 32>;
    case CFG_M: return &launch_generic<DT, EP, 128, 128, 64, 64>;
    default: break;
  }
  if constexpr (DT != F32) {
    switch (cfg) {
      case CFG_L: return &launch_dtl<DT, EP, 256, 256, 128, 64, 64, 2, PERSIST>;
      case CFG_LH: return &launch_dtl<DT, EP, 256, 256, 128, 64, 64, 2, LOCKSTEP_HALF>;
      case CFG_LM: return &launch_dtl<DT, EP, 128, 128, 32, 64, 64, 2, LOCKSTEP>;
      case CFG_LM4: return &launch_dtl<DT, EP, 128, 128, 64, 64, 64, 2, LOCKSTEP>;
      case CFG_LMD: return &launch_dtl<DT, EP, 128, 128, 32, 64, 64, 3, LOCKSTEP>;
      case CFG_L3: return &launch_dtl<DT, EP, 192, 256, 96, 64, 64, 2, PERSIST>;
      case CFG_LW: return &launch_dtl<DT, EP, 128, 256, 64, 64, 64, 2, PERSIST>;
      default: break;
    }
  }
  return nullptr;
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

// Operands stored transposed (LAY bit 0: A as (k,m), bit 1: B as (n,k)), 16-bit
// types: the configurations cfg_has_layouts names (the 256 x 256 tile persistent, with
// one workgroup per tile when the k loop does not suit the persistent kernel, or with
// copies on waves 0-3; the 128 x 128 tile).
template <int DT, int EP, int LAY>
LaunchFn pick_cfg_t(int cfg) {
  switch (cfg) {
    case CFG_L: return &launch_dtl<DT, EP, 256, 256, 128, 64, 64, 2, PERSIST, LAY>;
    case CFG_LH: return &launch_dtl<DT, EP, 256, 256, 128, 64, 64, 2, LOCKSTEP_HALF, LAY>;
    case CFG_LM: return &launch_dtl<DT, EP, 128, 128, 32, 64, 64, 2, LOCKSTEP, LAY>;
    case CFG_LMD: return &launch_dtl<DT, EP, 128, 128, 32, 64, 64, 3, LOCKSTEP, LAY>;
    default: return nullptr;
  }
}

template <int DT, int LAY>
LaunchFn pick_t(int ep, int cfg) {
  switch (ep) {
    case NONE: return pick_cfg_t<DT, NONE, LAY>(cfg);
    case RELU_BIAS: return pick_cfg_t<DT, RELU_BIAS, LAY>(cfg);
    case GELU_BIAS: return pick_cfg_t<DT, GELU_BIAS, LAY>(cfg);
    case RELU_AUX_BIAS: return pick_cfg_t<DT, RELU_AUX_BIAS, LAY>(cfg);
    case DRELU_BGRAD: return pick_cfg_t<DT, DRELU_BGRAD, LAY>(cfg);
    case BIAS: return pick_cfg_t<DT, BIAS, LAY>(cfg);
    default: return nullptr;
  }
}

// Defined one per storage type (and, for the transposed layouts, per layout), each in
// its own translation unit.
LaunchFn get_launch_f32(int ep, int cfg);
LaunchFn get_launch_f16(int ep, int cfg);
LaunchFn get_launch_bf16(int ep, int cfg);
LaunchFn get_launch_f16_lay1(int ep, int cfg);
LaunchFn get_launch_f16_lay2(int ep, int cfg);
LaunchFn get_launch_f16_lay3(int ep, int cfg);
LaunchFn get_launch_bf16_lay1(int ep, int cfg);
LaunchFn get_launch_bf16_lay2(int ep, int cfg);
LaunchFn get_launch_bf16_lay3(int ep, int cfg);

// Elementwise kernels of the unfused chains and the bgrad second pass.
hipError_t launch_bias_add(int dt, const void* in, const void* bias, int vec_dt, void* out, int64_t m, int n,
                           hipStream_t s);
hipError_t launch_relu(int dt, const void* in, void* out, int64_t m, int n, hipStream_t s);
hipError_t launch_bgrad_reduce(const float* partial, int t, int64_t m, void* bgrad, int vec_dt, hipStream_t s);
hipError_t launch_drelu(int dt, const void* in, const void* act, void* out, int64_t m, int n, hipStream_t s);
hipError_t launch_row_sum(int dt, const void* in, int64_t m, int n, void* bgrad, int vec_dt, hipStream_t s);

}  // namespace gek
