// Kernel-configuration table shared by the host runtime and the per-type
// instantiation units.
#pragma once

#include <hip/hip_runtime.h>

#include "gemm_dtl.hpp"
#include "gemm_generic.hpp"

namespace gek {

// Workgroup tile (BM x BN), wave tile (WM x WN), k-tile and LDS stages of each
// configuration. S and M use the register-staged kernel (any type); the L family
// uses the direct-to-LDS kernel (16-bit types only).
struct TileCfg {
  int bm, bn, wm, wn, bk, stages;
  const char* name;
  const char* loop;   // main loop of the direct-to-LDS kernels
};

enum CfgId { CFG_S = 0, CFG_M, CFG_L, CFG_LH, CFG_LA, CFG_LI, CFG_LS, CFG_LSH, CFG_LM, CFG_W4, CFG_W4S, CFG_P, CFG_LM4,
             CFG_COUNT };

constexpr TileCfg kTiles[CFG_COUNT] = {
    {64, 64, 32, 32, 0, 2, "S", ""},
    {128, 128, 64, 64, 0, 2, "M", ""},
    {256, 256, 128, 64, 64, 2, "L", "persistent lockstep interleaved, copies on waves 0-3"},   // 8 waves (default)
    {256, 256, 128, 64, 64, 2, "LH", "lockstep, copies on waves 0-3"},
    {256, 256, 128, 64, 64, 2, "LA", "lockstep"},
    {256, 256, 128, 64, 64, 2, "LI", "lockstep interleaved"},
    {256, 256, 128, 64, 32, 4, "LS", "lockstep spread interleaved"},
    {256, 256, 128, 64, 32, 4, "LSH", "lockstep spread interleaved, copies on waves 0-3"},
    {128, 128, 32, 64, 64, 2, "LM", "lockstep"},                        // 8 waves of 32 x 64, two per CU
    {256, 256, 128, 128, 64, 2, "W4", "lockstep"},                      // 4 waves of 128 x 128
    {256, 256, 128, 128, 32, 4, "W4S", "lockstep spread interleaved"},
    {256, 256, 128, 64, 32, 4, "P", "ping-pong"},                       // 8 waves in two groups
    {128, 128, 64, 64, 64, 2, "LM4", "lockstep"},                       // 4 waves of 64 x 64, two per CU
};

inline bool cfg_is_dtl(int c) { return c >= CFG_L; }
// Configurations whose kernel can split the last round's K loop (8-wave lockstep
// loops; the 4-wave tile has no registers left for the partial sums).
inline bool cfg_can_split(int c) { return c >= CFG_L && c <= CFG_LM; }

// Configurations with a persistent kernel, used when the tile grid is not split and
// k spans a whole number of stage rings, at least two.
inline bool cfg_can_persist(int c) { return c == CFG_L; }

using LaunchFn = hipError_t (*)(const Args&, int grid, hipStream_t);

template <int DT, int EP, int BM, int BN, int WM, int WN>
hipError_t launch_generic(const Args& a, int grid, hipStream_t s) {
  Args copy = a;
  void* params[] = {&copy};
  const void* fn = reinterpret_cast<const void*>(&gemm_epilog_kernel<DT, EP, BM, BN, WM, WN>);
  return hipLaunchKernel(fn, dim3(grid), dim3((BM / WM) * (BN / WN) * 64), params, 0, s);
}

// Main loop of a configuration: the lockstep loop's switches (interleaved reads,
// spread copies, copies on half the waves) or the ping-pong loop.
enum Loop { LOCKSTEP = 0, LOCKSTEP_ILV = 1, LOCKSTEP_SPREAD_ILV = 2, PINGPONG = 3, LOCKSTEP_HALF = 4,
            LOCKSTEP_SPREAD_ILV_HALF = 5, PERSIST = 6 };

// MFMAs of a k-tile's last step that the persistent loop issues before its barrier.
constexpr int kPersistPre = 4;

// LAY != 0 (an operand stored transposed): one workgroup per tile, plain lockstep loop.
template <int DT, int EP, int BM, int BN, int WM, int WN, int BK, int ST, int LOOP, int LAY = 0>
hipError_t launch_dtl(const Args& a, int grid, hipStream_t s) {
  Args copy = a;
  void* params[] = {&copy};
  const void* fn;
  constexpr bool SPREAD = LOOP == LOCKSTEP_SPREAD_ILV || LOOP == LOCKSTEP_SPREAD_ILV_HALF;
  constexpr bool ILV = LOOP == LOCKSTEP_ILV || LOOP == PERSIST || SPREAD;
  constexpr int CW = (LOOP == LOCKSTEP_HALF || LOOP == LOCKSTEP_SPREAD_ILV_HALF || LOOP == PERSIST)
                         ? (BM / WM) * (BN / WN) / 2 : 0;
  if constexpr (LAY != 0) {
    static_assert(LOOP == LOCKSTEP || LOOP == LOCKSTEP_HALF || LOOP == PERSIST,
                  "transposed operands: plain lockstep loop or the persistent kernel");
    fn = reinterpret_cast<const void*>(&gemm_dtl_kernel<DT, EP, BM, BN, WM, WN, BK, ST, false, false, CW, LAY>);
    if constexpr (LOOP == PERSIST) {
      if (a.persist_grid > 0) {
        fn = reinterpret_cast<const void*>(&gemm_persist_kernel<DT, EP, BM, BN, WM, WN, BK, ST, CW, kPersistPre, LAY>);
        grid = a.persist_grid;
      }
    }
  } else if constexpr (LOOP == PINGPONG) {
    fn = reinterpret_cast<const void*>(&gemm_pp_kernel<DT, EP, BM, BN, WM, WN, BK, ST>);
  } else {
    fn = reinterpret_cast<const void*>(&gemm_dtl_kernel<DT, EP, BM, BN, WM, WN, BK, ST, SPREAD, ILV, CW>);
    if constexpr ((BM / WM) * (BN / WN) == 8) {   // the split tail exists for the 8-wave tiles
      if (a.dp_tiles < grid) {
        fn = reinterpret_cast<const void*>(&gemm_sk_kernel<DT, EP, BM, BN, WM, WN, BK, ST, SPREAD, ILV, CW>);
        grid = a.dp_tiles + a.sk_wgs;
      }
    }
    if constexpr (LOOP == PERSIST) {
      if (a.dp_tiles == grid && a.persist_grid > 0) {
        fn = reinterpret_cast<const void*>(&gemm_persist_kernel<DT, EP, BM, BN, WM, WN, BK, ST, CW, kPersistPre>);
        grid = a.persist_grid;
      }
    }
  }
  return hipLaunchKernel(fn, dim3(grid), dim3((BM / WM) * (BN / WN) * 64), params, 0, s);
}

// Partial-accumulator bytes of one split workgroup of a configuration (one tile, fp32).
inline size_t sk_slot_bytes(const TileCfg& c) { return (size_t)c.bm * c.bn * sizeof(float); }

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
      case CFG_LA: return &launch_dtl<DT, EP, 256, 256, 128, 64, 64, 2, LOCKSTEP>;
      case CFG_LI: return &launch_dtl<DT, EP, 256, 256, 128, 64, 64, 2, LOCKSTEP_ILV>;
      case CFG_LS: return &launch_dtl<DT, EP, 256, 256, 128, 64, 32, 4, LOCKSTEP_SPREAD_ILV>;
      case CFG_LSH: return &launch_dtl<DT, EP, 256, 256, 128, 64, 32, 4, LOCKSTEP_SPREAD_ILV_HALF>;
      case CFG_LM: return &launch_dtl<DT, EP, 128, 128, 32, 64, 64, 2, LOCKSTEP>;
      case CFG_W4: return &launch_dtl<DT, EP, 256, 256, 128, 128, 64, 2, LOCKSTEP>;
      case CFG_W4S: return &launch_dtl<DT, EP, 256, 256, 128, 128, 32, 4, LOCKSTEP_SPREAD_ILV>;
      case CFG_P: return &launch_dtl<DT, EP, 256, 256, 128, 64, 32, 4, PINGPONG>;
      case CFG_LM4: return &launch_dtl<DT, EP, 128, 128, 64, 64, 64, 2, LOCKSTEP>;
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
// types: the 256 x 256 tile persistent (L; one workgroup per tile when the k loop does
// not suit the persistent kernel) or with copies on waves 0-3 (LH), or the 128 x 128
// tile (LM).
inline bool cfg_has_layouts(int c) { return c == CFG_L || c == CFG_LH || c == CFG_LM; }

template <int DT, int EP, int LAY>
LaunchFn pick_cfg_t(int cfg) {
  switch (cfg) {
    case CFG_L: return &launch_dtl<DT, EP, 256, 256, 128, 64, 64, 2, PERSIST, LAY>;
    case CFG_LH: return &launch_dtl<DT, EP, 256, 256, 128, 64, 64, 2, LOCKSTEP_HALF, LAY>;
    case CFG_LM: return &launch_dtl<DT, EP, 128, 128, 32, 64, 64, 2, LOCKSTEP, LAY>;
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

// Elementwise kernels of the unfused chain and the bgrad second pass.
hipError_t launch_bias_add(int dt, const void* in, const void* bias, int vec_dt, void* out, int64_t m, int n,
                           hipStream_t s);
hipError_t launch_relu(int dt, const void* in, void* out, int64_t m, int n, hipStream_t s);
hipError_t launch_bgrad_reduce(const float* partial, int t, int64_t m, void* bgrad, int vec_dt, hipStream_t s);

}  // namespace gek
