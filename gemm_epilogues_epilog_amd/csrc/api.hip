// Host runtime of the fused GEMM + epilogue library: argument validation, plan
// (kernel configuration + workspace), execute (launches on the caller's stream),
// free. The C ABI is declared in include/gemm_epilog.h.
//
// The plan / execute / free split follows the stateful matmul object of
// "Dissecting nvmath-python: a seamless bridge between NumPy and cuBLASLt"
// (blog.hotdry.top), paragraph on the plan-execute-free lifecycle, and
// "nvmath-python wraps cuBLASLt" (blog.hotdry.top), body: planning is the costly
// step done once, execution is light and repeated.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <string>
#include <utility>
#include <vector>

#include "gemm_epilog.h"
#include "launch.hpp"
#include "plan_host.hpp"

struct ge_plan {
  int64_t m;
  int n, k;
  ge_dtypes_t dt;
  ge_epilog_t ep;
  int device;
  int cus;                 // compute units of the device
  bool allow_split, allow_persist;
  geh::Layout L;           // configuration, grid, split tail, workspace layout
  gek::LaunchFn gemm;      // main kernel (the NONE instance for the unfused chain)
  void* ws;                // device workspace
  uint32_t epoch;          // execute counter, 1 .. 2^31 - 1
  uint32_t spin_limit;     // polls of a split-tail owner's bounded wait
  std::string desc;
};

namespace {

// Default polls of a split-tail owner's wait for a partial (about a second);
// GE_SK_SPIN=n overrides it (failure-path tests force a wait to run out).
constexpr uint32_t kSkSpinDefault = 1u << 20;

// Zero `bytes` of device memory and wait for it, on a stream of its own (default
// priority) so that other streams are not synchronised.
hipError_t clear_now(void* p, size_t bytes) {
  hipStream_t st = nullptr;
  hipError_t e = hipStreamCreateWithFlags(&st, hipStreamNonBlocking);
  if (e != hipSuccess) return e;
  e = hipMemsetAsync(p, 0, bytes, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  const hipError_t d = hipStreamDestroy(st);
  return e != hipSuccess ? e : d;
}

static_assert((int)gek::NONE == GE_EPILOG_NONE && (int)gek::RELU_BIAS == GE_EPILOG_RELU_BIAS &&
                  (int)gek::GELU_BIAS == GE_EPILOG_GELU_BIAS && (int)gek::RELU_AUX_BIAS == GE_EPILOG_RELU_AUX_BIAS &&
                  (int)gek::DRELU_BGRAD == GE_EPILOG_DRELU_BGRAD && (int)gek::BIAS == GE_EPILOG_BIAS,
              "the kernels' epilogue codes are the public ones");

gek::LaunchFn lookup(ge_dtype_t ab, int ep, int cfg, int lay) {
  if (lay != 0 && !gek::cfg_has_layouts(cfg)) return nullptr;
  switch (ab) {
    case GE_F32: return lay == 0 ? gek::get_launch_f32(ep, cfg) : nullptr;
    case GE_F16:
      switch (lay) {
        case 0: return gek::get_launch_f16(ep, cfg);
        case 1: return gek::get_launch_f16_lay1(ep, cfg);
        case 2: return gek::get_launch_f16_lay2(ep, cfg);
        case 3: return gek::get_launch_f16_lay3(ep, cfg);
      }
      break;
    case GE_BF16:
      switch (lay) {
        case 0: return gek::get_launch_bf16(ep, cfg);
        case 1: return gek::get_launch_bf16_lay1(ep, cfg);
        case 2: return gek::get_launch_bf16_lay2(ep, cfg);
        case 3: return gek::get_launch_bf16_lay3(ep, cfg);
      }
      break;
  }
  return nullptr;
}

// A plan for a validated problem with a given tile configuration; allow_split and
// allow_persist permit the split tail and the persistent kernel where they apply.
ge_status_t build_plan(int64_t m, int64_t n, int64_t k, ge_dtypes_t dt, ge_epilog_t ep, int lay, int dev, int cus,
                       int cfg, bool allow_split, bool allow_persist, ge_handle_t* out) {
  geh::Layout L;
  if (ge_status_t st = geh::make_layout(m, n, k, dt, ep, lay, cus, cfg, allow_split, allow_persist, &L); st != GE_OK)
    return st;
  gek::LaunchFn fn = lookup(dt.ab, geh::gemm_epilog_of(ep), cfg, lay);
  if (!fn) return GE_ERR_NOT_SUPPORTED;
  ge_plan* h = new (std::nothrow) ge_plan();
  if (!h) return GE_ERR_ALLOC;
  h->m = m;
  h->n = (int)n;
  h->k = (int)k;
  h->dt = dt;
  h->ep = ep;
  h->device = dev;
  h->cus = cus;
  h->allow_split = allow_split;
  h->allow_persist = allow_persist;
  h->L = L;
  h->gemm = fn;
  h->spin_limit = kSkSpinDefault;
  if (const char* e = std::getenv("GE_SK_SPIN")) {
    const long v = std::atol(e);
    if (v >= 0 && v <= (long)kSkSpinDefault) h->spin_limit = (uint32_t)v;
  }
  if (L.ws_bytes) {
    if (hipMalloc(&h->ws, L.ws_bytes) != hipSuccess) {
      delete h;
      return GE_ERR_ALLOC;
    }
    // split flags start at 0 (idle), the lost-wait count after them too; cleared on a
    // stream of the plan's own and waited for, so no other stream is held up
    if (L.sk_wgs && clear_now(static_cast<char*>(h->ws) + L.off_sk_flag, L.sk_flag_bytes) != hipSuccess) {
      hipFree(h->ws);
      delete h;
      return GE_ERR_HIP;
    }
  }
  h->desc = geh::describe(dt, ep, L);
  if (const char* lg = std::getenv("GE_LOG"); lg && lg[0] == '1')
    std::fprintf(stderr, "gemm_epilog_plan: m=%lld n=%lld k=%lld -> %s, workspace %zu bytes\n", (long long)m,
                 (long long)n, (long long)k, h->desc.c_str(), L.ws_bytes);
  *out = h;
  return GE_OK;
}

// Enqueue one execute of plan h with its workspace at `ws` (arguments already checked):
// the main kernel, then the bgrad second pass or the unfused chain's elementwise kernels.
ge_status_t enqueue(const ge_plan& h, char* ws, uint32_t epoch, const void* A, const void* B, const void* bias,
                    void* D, void* aux, void* bgrad, hipStream_t s) {
  const geh::Layout& L = h.L;
  gek::Args a;
  a.A = A;
  a.B = B;
  a.bias = bias;
  void* t1 = ws + L.off_t1;
  void* t2 = ws + L.off_t2;
  float* partial = reinterpret_cast<float*>(ws + L.off_partial);
  a.D = geh::is_unfused(h.ep) ? t1 : D;
  a.aux = static_cast<uint32_t*>(aux);
  a.partial = h.ep == GE_EPILOG_DRELU_BGRAD ? partial : nullptr;
  a.m = h.m;
  a.n = h.n;
  a.k = h.k;
  a.vec_dt = (int)h.dt.vec;
  a.tiles_m = L.tiles_m;
  a.tiles_n = L.tiles_n;
  a.group_m = L.group_m;
  a.dp_tiles = L.dp_tiles;
  a.sk_units = L.sk_units;
  a.sk_wgs = L.sk_wgs;
  a.sk_partial = L.sk_wgs ? reinterpret_cast<float*>(ws + L.off_sk_partial) : nullptr;
  a.sk_flag = L.sk_wgs ? reinterpret_cast<uint32_t*>(ws + L.off_sk_flag) : nullptr;
  a.sk_spin_limit = h.spin_limit;
  a.persist_grid = L.persist_grid;
  a.epoch = epoch;
  if (h.gemm(a, L.tiles_m * L.tiles_n, s) != hipSuccess) return GE_ERR_HIP;
  if (h.ep == GE_EPILOG_DRELU_BGRAD) {
    if (gek::launch_bgrad_reduce(partial, L.partial_cols, h.m, bgrad, (int)h.dt.vec, s) != hipSuccess)
      return GE_ERR_HIP;
  } else if (h.ep == GE_EPILOG_RELU_BIAS_UNFUSED) {
    if (gek::launch_bias_add((int)h.dt.d, t1, bias, (int)h.dt.vec, t2, h.m, h.n, s) != hipSuccess) return GE_ERR_HIP;
    if (gek::launch_relu((int)h.dt.d, t2, D, h.m, h.n, s) != hipSuccess) return GE_ERR_HIP;
  } else if (h.ep == GE_EPILOG_DRELU_BGRAD_UNFUSED) {
    if (gek::launch_drelu((int)h.dt.d, t1, aux, D, h.m, h.n, s) != hipSuccess) return GE_ERR_HIP;
    if (gek::launch_row_sum((int)h.dt.d, D, h.m, h.n, bgrad, (int)h.dt.vec, s) != hipSuccess) return GE_ERR_HIP;
  }
  return GE_OK;
}

// The device the caller has current, if it is a gfx950; its compute units.
ge_status_t query_device(int* dev, int* cus) {
  if (hipGetDevice(dev) != hipSuccess) return GE_ERR_HIP;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, *dev) != hipSuccess) return GE_ERR_HIP;
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return GE_ERR_NOT_SUPPORTED;
  *cus = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 256;
  return GE_OK;
}

// ---- the static scratch of gemm_epilog_execute_noalloc ----
// Each device that runs this code object holds its own copy of `scratch`. In host code
// the name stands for the host-side shadow of the variable, not for device memory:
// only the address that hipGetSymbolAddress returns, per device, is used.
constexpr size_t kScratchBytes = GEMM_EPILOG_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
struct ScratchState {
  std::mutex mu;
  void* ptr[kMaxDevices] = {};       // device address of `scratch` per device
  int cus[kMaxDevices] = {};         // compute units per device (0: not yet queried)
  uint32_t epoch[kMaxDevices] = {};  // execute counter per device
};
ScratchState g_scratch;

}  // namespace

namespace gek {
// Zeroes n words (the split tail's flags in the static scratch); a kernel rather than a
// memset, so that it may also sit in a captured graph.
__global__ void clear_words_kernel(uint32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}
}  // namespace gek

extern "C" {

const char* gemm_epilog_status_string(ge_status_t s) {
  switch (s) {
    case GE_OK: return "GE_OK";
    case GE_ERR_INVALID_VALUE: return "GE_ERR_INVALID_VALUE: a size or enum value is out of range";
    case GE_ERR_NOT_SUPPORTED: return "GE_ERR_NOT_SUPPORTED: dtype combination or shape not supported";
    case GE_ERR_NULL_POINTER: return "GE_ERR_NULL_POINTER: a required pointer is NULL";
    case GE_ERR_MISALIGNED: return "GE_ERR_MISALIGNED: a pointer violates its alignment rule";
    case GE_ERR_ALLOC: return "GE_ERR_ALLOC: allocation failed";
    case GE_ERR_HIP: return "GE_ERR_HIP: a HIP runtime call failed";
    case GE_ERR_SCRATCH:
      return "GE_ERR_SCRATCH: the problem needs more workspace than the 64 MiB static scratch of "
             "gemm_epilog_execute_noalloc";
  }
  return "unknown status";
}

size_t gemm_epilog_aux_bytes(int64_t m, int64_t n) {
  if (m < 1 || n < 1) return 0;
  return (size_t)4 * (size_t)((m + 31) / 32) * (size_t)n;
}

ge_status_t gemm_epilog_plan(int64_t m, int64_t n, int64_t k, ge_dtypes_t dt, ge_epilog_t ep, ge_handle_t* out) {
  return gemm_epilog_plan_ex(m, n, k, dt, ep, GE_OP_N, GE_OP_N, out);
}

ge_status_t gemm_epilog_plan_ex(int64_t m, int64_t n, int64_t k, ge_dtypes_t dt, ge_epilog_t ep, ge_op_t op_a,
                                ge_op_t op_b, ge_handle_t* out) {
  // host-only validation: no HIP call before it passes
  if (!out) return GE_ERR_NULL_POINTER;
  int lay = 0;
  if (ge_status_t st = geh::check_plan_args(m, n, k, dt, ep, op_a, op_b, &lay); st != GE_OK) return st;
  int dev = 0, cus = 0;
  if (ge_status_t st = query_device(&dev, &cus); st != GE_OK) return st;
  return build_plan(m, n, k, dt, ep, lay, dev, cus, geh::choose_cfg(m, n, k, dt.ab, cus, lay),
                    !geh::env_off("GE_STREAMK"), !geh::env_off("GE_PERSIST"), out);
}

ge_status_t gemm_epilog_execute(ge_handle_t h, const void* A, const void* B, const void* bias, void* D, void* aux,
                                void* bgrad, void* stream) {
  // host-only validation
  if (!h) return GE_ERR_NULL_POINTER;
  if (ge_status_t st = geh::check_execute_args(h->ep, h->dt, A, B, bias, D, aux, bgrad); st != GE_OK) return st;
  h->epoch = h->epoch % 0x7fffffffu + 1u;
  return enqueue(*h, static_cast<char*>(h->ws), h->epoch, A, B, bias, D, aux, bgrad, static_cast<hipStream_t>(stream));
}

ge_status_t gemm_epilog_autotune(ge_handle_t h, const void* A, const void* B, const void* bias, void* D, void* aux,
                                 void* bgrad, void* stream, int repeats, float* best_ms) {
  if (!h) return GE_ERR_NULL_POINTER;
  if (repeats < 1 || repeats > 1000) return GE_ERR_INVALID_VALUE;
  // the argument rules of execute, checked once on the plan itself before any timing
  if (ge_status_t st = gemm_epilog_execute(h, A, B, bias, D, aux, bgrad, stream); st != GE_OK) return st;

  // Candidates: every configuration the plan's types and operand layout can run, with
  // and without the split tail; the persistent kernel wherever it applies.
  struct Cand {
    int cfg;
    bool split, persist;
  };
  std::vector<Cand> cands;
  if (h->dt.ab == GE_F32) {
    cands = {{gek::CFG_S, false, false}, {gek::CFG_M, false, false}};
  } else if (h->L.lay != 0) {
    cands = {{gek::CFG_L, false, true}, {gek::CFG_L, false, false}, {gek::CFG_LH, false, false},
             {gek::CFG_LM, false, false}, {gek::CFG_LMD, false, false}};
  } else {
    cands = {{gek::CFG_L, true, true},   {gek::CFG_L, false, true},   {gek::CFG_L, false, false},
             {gek::CFG_L3, true, true},  {gek::CFG_L3, false, true},  {gek::CFG_LW, true, true},
             {gek::CFG_LW, false, true},
             {gek::CFG_LH, true, false}, {gek::CFG_LH, false, false}, {gek::CFG_LM, true, false},
             {gek::CFG_LM, false, false}, {gek::CFG_LM4, false, false}, {gek::CFG_LMD, true, false},
             {gek::CFG_LMD, false, false}};
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
    if (e0) hipEventDestroy(e0);
    return GE_ERR_HIP;
  }
  // time one plan: one warm-up execute, then `repeats` between two events
  auto time_plan = [&](ge_plan* c, float* ms) -> ge_status_t {
    if (ge_status_t st = gemm_epilog_execute(c, A, B, bias, D, aux, bgrad, stream); st != GE_OK) return st;
    if (hipEventRecord(e0, s) != hipSuccess) return GE_ERR_HIP;
    for (int r = 0; r < repeats; ++r)
      if (ge_status_t st = gemm_epilog_execute(c, A, B, bias, D, aux, bgrad, stream); st != GE_OK) return st;
    if (hipEventRecord(e1, s) != hipSuccess || hipEventSynchronize(e1) != hipSuccess) return GE_ERR_HIP;
    return hipEventElapsedTime(ms, e0, e1) == hipSuccess ? GE_OK : GE_ERR_HIP;
  };

  ge_status_t st = GE_OK;
  float best = 0.0f;
  if ((st = time_plan(h, &best)) != GE_OK) {
    hipEventDestroy(e0);
    hipEventDestroy(e1);
    return st;
  }
  ge_plan* winner = nullptr;   // a better plan than h, if one is found
  std::vector<std::string> seen = {h->desc};
  for (const Cand& c : cands) {
    ge_handle_t t = nullptr;
    if (build_plan(h->m, h->n, h->k, h->dt, h->ep, h->L.lay, h->device, h->cus, c.cfg, c.split, c.persist, &t) !=
        GE_OK)
      continue;   // e.g. no workspace for this configuration: not a candidate
    if (std::find(seen.begin(), seen.end(), t->desc) != seen.end()) {   // the same kernels as one timed already
      gemm_epilog_free(t);
      continue;
    }
    seen.push_back(t->desc);
    float ms = 0.0f;
    if ((st = time_plan(t, &ms)) != GE_OK) {
      gemm_epilog_free(t);
      break;
    }
    if (ms < best) {
      best = ms;
      if (winner) gemm_epilog_free(winner);
      winner = t;
    } else {
      gemm_epilog_free(t);
    }
  }
  hipEventDestroy(e0);
  hipEventDestroy(e1);
  if (st != GE_OK) {
    if (winner) gemm_epilog_free(winner);
    return st;
  }
  if (winner) {
    // the stream is idle (every timing ended with an event synchronisation): the plan
    // takes the winner's configuration and workspace, the winner's struct the old ones
    std::swap(*h, *winner);
    gemm_epilog_free(winner);
    // leave the outputs as an execute of the chosen configuration writes them
    if ((st = gemm_epilog_execute(h, A, B, bias, D, aux, bgrad, stream)) != GE_OK) return st;
  }
  if (best_ms) *best_ms = best / (float)repeats;
  return GE_OK;
}

ge_status_t gemm_epilog_execute_noalloc(int64_t m, int64_t n, int64_t k, ge_dtypes_t dt, ge_epilog_t ep,
                                        ge_op_t op_a, ge_op_t op_b, const void* A, const void* B, const void* bias,
                                        void* D, void* aux, void* bgrad, void* stream) {
  // host-only validation first, as for plan_ex and execute
  int lay = 0;
  if (ge_status_t st = geh::check_plan_args(m, n, k, dt, ep, op_a, op_b, &lay); st != GE_OK) return st;
  if (ge_status_t st = geh::check_execute_args(ep, dt, A, B, bias, D, aux, bgrad); st != GE_OK) return st;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return GE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return GE_ERR_NOT_SUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);

  // once per device: the device's address of the scratch, its compute units, and its
  // flag words cleared on this stream (ahead of this call's kernels)
  char* ws = nullptr;
  int cus = 0;
  uint32_t epoch = 0;
  {
    std::lock_guard<std::mutex> lock(g_scratch.mu);
    if (!g_scratch.ptr[dev]) {
      int c = 0;
      if (ge_status_t st = query_device(&dev, &c); st != GE_OK) return st;
      void* p = nullptr;
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return GE_ERR_HIP;
      uint32_t* words = static_cast<uint32_t*>(p);
      int nw = gek::kSkFlagWords;
      void* params[] = {&words, &nw};
      if (hipLaunchKernel(reinterpret_cast<const void*>(&gek::clear_words_kernel), dim3(gek::kSkFlagWords / 256),
                          dim3(256), params, 0, s) != hipSuccess)
        return GE_ERR_HIP;
      g_scratch.ptr[dev] = p;
      g_scratch.cus[dev] = c;
    }
    ws = static_cast<char*>(g_scratch.ptr[dev]);
    cus = g_scratch.cus[dev];
    g_scratch.epoch[dev] = g_scratch.epoch[dev] % 0x7fffffffu + 1u;
    epoch = g_scratch.epoch[dev];
  }

  // the plan, on the stack: the table's configuration; without the split tail when its
  // partials do not fit the scratch
  const int cfg = geh::choose_cfg(m, n, k, dt.ab, cus, lay);
  const bool persist = !geh::env_off("GE_PERSIST");
  geh::Layout L;
  if (ge_status_t st = geh::make_layout(m, n, k, dt, ep, lay, cus, cfg, !geh::env_off("GE_STREAMK"), persist, &L);
      st != GE_OK)
    return st;
  if (L.ws_bytes > kScratchBytes &&
      geh::make_layout(m, n, k, dt, ep, lay, cus, cfg, false, persist, &L) != GE_OK)
    return GE_ERR_NOT_SUPPORTED;
  if (L.ws_bytes > kScratchBytes) return GE_ERR_SCRATCH;
  ge_plan h;
  h.m = m;
  h.n = (int)n;
  h.k = (int)k;
  h.dt = dt;
  h.ep = ep;
  h.device = dev;
  h.cus = cus;
  h.L = L;
  h.gemm = lookup(dt.ab, geh::gemm_epilog_of(ep), cfg, lay);
  if (!h.gemm) return GE_ERR_NOT_SUPPORTED;
  h.ws = ws;
  h.spin_limit = kSkSpinDefault;
  if (const char* e = std::getenv("GE_SK_SPIN")) {
    const long v = std::atol(e);
    if (v >= 0 && v <= (long)kSkSpinDefault) h.spin_limit = (uint32_t)v;
  }
  return enqueue(h, ws, epoch, A, B, bias, D, aux, bgrad, s);
}

ge_status_t gemm_epilog_lost_waits(ge_handle_t h, void* stream, uint32_t* count) {
  if (!h || !count) return GE_ERR_NULL_POINTER;
  *count = 0;
  if (h->L.sk_wgs == 0) return GE_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t* word = reinterpret_cast<uint32_t*>(static_cast<char*>(h->ws) + h->L.off_sk_flag) + gek::kSkLostWord;
  uint32_t v = 0;
  if (hipMemcpyAsync(&v, word, sizeof(v), hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipMemsetAsync(word, 0, sizeof(v), s) != hipSuccess || hipStreamSynchronize(s) != hipSuccess)
    return GE_ERR_HIP;
  *count = v;
  return GE_OK;
}

ge_status_t gemm_epilog_free(ge_handle_t h) {
  if (!h) return GE_OK;
  ge_status_t st = GE_OK;
  if (h->ws && hipFree(h->ws) != hipSuccess) st = GE_ERR_HIP;
  delete h;
  return st;
}

size_t gemm_epilog_workspace_bytes(ge_handle_t h) { return h ? h->L.ws_bytes : 0; }

const char* gemm_epilog_describe(ge_handle_t h) { return h ? h->desc.c_str() : ""; }

}  // extern "C"

namespace gek {

// ---- second pass of DRELU_BGRAD: bgrad[i] = sum over t of partial[t][i] ----
// A workgroup of 4 waves takes 64 rows, one per lane; wave w sums the t-range
// [w T/4, (w+1) T/4) in ascending order with 16 loads in flight, and wave 0 adds the
// four range sums in order w = 0 .. 3. The order is fixed, so results repeat bit for
// bit; there are no atomics.
constexpr int kReduceWaves = 4, kReduceBatch = 16;
__global__ __launch_bounds__(64 * kReduceWaves) void bgrad_reduce_kernel(const float* __restrict__ partial, int T,
                                                                       int64_t M, void* bgrad, int vec_dt) {
  __shared__ float sums[kReduceWaves][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t i = (int64_t)blockIdx.x * 64 + lane;
  const int t0 = (int)((int64_t)T * w / kReduceWaves), t1 = (int)((int64_t)T * (w + 1) / kReduceWaves);
  float s = 0.0f;
  if (i < M) {
    for (int t = t0; t < t1; t += kReduceBatch) {
      float v[kReduceBatch];
#pragma unroll
      for (int j = 0; j < kReduceBatch; ++j) v[j] = t + j < t1 ? partial[(int64_t)(t + j) * M + i] : 0.0f;
#pragma unroll
      for (int j = 0; j < kReduceBatch; ++j) s += v[j];
    }
  }
  sums[w][lane] = s;
  __syncthreads();
  if (w == 0 && i < M) {
    float r = sums[0][lane];
#pragma unroll
    for (int q = 1; q < kReduceWaves; ++q) r += sums[q][lane];
    store_vec(bgrad, vec_dt, i, r);
  }
}

hipError_t launch_bias_add(int dt, const void* in, const void* bias, int vec_dt, void* out, int64_t m, int n,
                           hipStream_t s) {
  const int E = dt == F32 ? 4 : 8;
  const int64_t chunks = m * (int64_t)n / E;
  const dim3 grid((unsigned)((chunks + 255) / 256));
  void* params[] = {&in, &bias, &vec_dt, &out, const_cast<int64_t*>(&chunks), &n};
  const void* fn = dt == F32 ? reinterpret_cast<const void*>(&bias_add_kernel<F32>)
                 : dt == F16 ? reinterpret_cast<const void*>(&bias_add_kernel<F16>)
                             : reinterpret_cast<const void*>(&bias_add_kernel<BF16>);
  return hipLaunchKernel(fn, grid, dim3(256), params, 0, s);
}

hipError_t launch_relu(int dt, const void* in, void* out, int64_t m, int n, hipStream_t s) {
  const int E = dt == F32 ? 4 : 8;
  const int64_t chunks = m * (int64_t)n / E;
  const dim3 grid((unsigned)((chunks + 255) / 256));
  void* params[] = {&in, &out, const_cast<int64_t*>(&chunks)};
  const void* fn = dt == F32 ? reinterpret_cast<const void*>(&relu_kernel<F32>)
                 : dt == F16 ? reinterpret_cast<const void*>(&relu_kernel<F16>)
                             : reinterpret_cast<const void*>(&relu_kernel<BF16>);
  return hipLaunchKernel(fn, grid, dim3(256), params, 0, s);
}

hipError_t launch_drelu(int dt, const void* in, const void* act, void* out, int64_t m, int n, hipStream_t s) {
  const int E = dt == F32 ? 4 : 8;
  const int64_t chunks = m * (int64_t)n / E;
  const dim3 grid((unsigned)((chunks + 255) / 256));
  void* params[] = {&in, &act, &out, const_cast<int64_t*>(&chunks)};
  const void* fn = dt == F32 ? reinterpret_cast<const void*>(&drelu_kernel<F32>)
                 : dt == F16 ? reinterpret_cast<const void*>(&drelu_kernel<F16>)
                             : reinterpret_cast<const void*>(&drelu_kernel<BF16>);
  return hipLaunchKernel(fn, grid, dim3(256), params, 0, s);
}

hipError_t launch_row_sum(int dt, const void* in, int64_t m, int n, void* bgrad, int vec_dt, hipStream_t s) {
  const dim3 grid((unsigned)((m + 3) / 4));
  void* params[] = {&in, &m, &n, &bgrad, &vec_dt};
  const void* fn = dt == F32 ? reinterpret_cast<const void*>(&row_sum_kernel<F32>)
                 : dt == F16 ? reinterpret_cast<const void*>(&row_sum_kernel<F16>)
                             : reinterpret_cast<const void*>(&row_sum_kernel<BF16>);
  return hipLaunchKernel(fn, grid, dim3(256), params, 0, s);
}

hipError_t launch_bgrad_reduce(const float* partial, int t, int64_t m, void* bgrad, int vec_dt, hipStream_t s) {
  const dim3 grid((unsigned)((m + 63) / 64));
  void* params[] = {&partial, &t, &m, &bgrad, &vec_dt};
  return hipLaunchKernel(reinterpret_cast<const void*>(&bgrad_reduce_kernel), grid, dim3(64 * kReduceWaves), params,
                         0, s);
}

}  // namespace gek
