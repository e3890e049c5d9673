// Host-side plan arithmetic of the fused GEMM + epilogue library: argument
// validation, the tile-configuration choice, the split tail of a sparse last round,
// the persistent grid and the workspace layout. Plain C++17 with no HIP call or
// header, so it also builds with g++ (the CPU tests run it under AddressSanitizer and
// UndefinedBehaviorSanitizer). The HIP runtime (api.hip) allocates and launches what
// this unit decides.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>

#include "gemm_epilog.h"

namespace geh {

// Bytes of the split tail's flag region at the start of a workspace (gek::kSkFlagWords
// words: the flags, then the count of owner waits that ran out in the last word).
constexpr size_t kSkFlagRegion = 4096;

// Everything a plan decides before it touches a device.
struct Layout {
  int cfg = 0;            // gek::CfgId
  int lay = 0;            // operand storage: bit 0 A as (k,m), bit 1 B as (n,k)
  int tiles_m = 0, tiles_n = 0;
  int group_m = 8;        // m-tiles per group of the tile order
  int dp_tiles = 0;       // tiles computed whole (all tiles when the grid is not split)
  int sk_units = 0;       // split tail: k-tiles per split workgroup
  int sk_wgs = 0;         // split tail: split workgroups
  int sk_parts = 0;       // split tail: runs per tile when they cover whole tiles (each finishes a part), else 0
  int persist_grid = 0;   // persistent workgroups (0: one workgroup per tile)
  int partial_cols = 0;   // DRELU_BGRAD: partial row sums per row (one per wave column)
  // Workspace: [split flags][DRELU_BGRAD partials | unfused T1, T2][split partials];
  // the flags, the partials and T1 start 256-byte aligned, T2 16-byte aligned. Offsets
  // are meaningful when the region exists.
  size_t off_partial = 0, off_t1 = 0, off_t2 = 0, off_sk_partial = 0, off_sk_flag = 0;
  size_t sk_flag_bytes = 0;
  size_t ws_bytes = 0;
};

size_t elem_size(ge_dtype_t d);
bool uses_bias(ge_epilog_t e);
// k-tiles per run when `rem` sparse tiles of `kt` k-tiles share `cus` compute units
// (before the GE_SK_RUN override).
int64_t split_run_length(int64_t rem, int64_t kt, int cus);
// The unfused baselines: a product kernel without epilogue into T1, then kernels of
// their own for the remaining steps.
bool is_unfused(ge_epilog_t e);
// The epilogue the product kernel applies (the kernels' codes equal the public enum's):
// NONE for the unfused baselines, the plan's own otherwise.
int gemm_epilog_of(ge_epilog_t e);

// The argument rules of gemm_epilog_plan_ex; on GE_OK *lay holds the storage bits.
ge_status_t check_plan_args(int64_t m, int64_t n, int64_t k, ge_dtypes_t dt, ge_epilog_t ep, ge_op_t op_a,
                            ge_op_t op_b, int* lay);

// The configuration the plan takes on a device with `cus` compute units (GE_TILE may
// force one).
int choose_cfg(int64_t m, int64_t n, int64_t k, ge_dtype_t ab, int cus, int lay);

// Grid, split tail, persistent grid and workspace of a validated problem with a given
// configuration; GE_ERR_NOT_SUPPORTED when the configuration cannot run it.
ge_status_t make_layout(int64_t m, int64_t n, int64_t k, ge_dtypes_t dt, ge_epilog_t ep, int lay, int cus, int cfg,
                        bool allow_split, bool allow_persist, Layout* out);

// The plan's human-readable configuration (gemm_epilog_describe).
std::string describe(ge_dtypes_t dt, ge_epilog_t ep, const Layout& L);

// The pointer rules of gemm_epilog_execute.
ge_status_t check_execute_args(ge_epilog_t ep, ge_dtypes_t dt, const void* A, const void* B, const void* bias,
                               const void* D, const void* aux, const void* bgrad);

// An environment switch set to "0" (tuning experiments).
bool env_off(const char* name);

}  // namespace geh
