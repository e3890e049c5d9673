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
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <string>
#include <utility>
#include <vector>

#include "gemm_epilog.h"
#include "launch.hpp"

struct ge_plan {
  int64_t m;
  int n, k;
  ge_dtypes_t dt;
  ge_epilog_t ep;
  int cfg;                 // gek::CfgId
  int lay;                 // operand storage: bit 0 A as (k,m), bit 1 B as (n,k)
  int device;
  int tiles_m, tiles_n, group_m;
  gek::LaunchFn gemm;      // main kernel (the NONE instance for the unfused chain)
  void* ws;                // device workspace
  size_t ws_bytes;
  float* partial;          // DRELU_BGRAD per-wave row sums
  int partial_cols;
  void* t1;                // unfused intermediates
  void* t2;
  int dp_tiles;            // split tail: tiles computed whole (all tiles when not split)
  int sk_units, sk_wgs;    // split tail: k-tiles per split workgroup, split workgroups
  float* sk_partial;       // split tail: one fp32 tile per split workgroup
  uint32_t* sk_flag;       // split tail: epoch of each published partial
  int persist_grid = 0;    // persistent workgroups (0: one workgroup per tile)
  int cus;                 // compute units of the device
  bool allow_split, allow_persist;
  uint32_t epoch;          // execute counter, 1 .. 2^31 - 1
  std::string desc;
};

namespace {

size_t elem_size(ge_dtype_t d) { return d == GE_F32 ? 4 : 2; }

bool known_dtype(int d) { return d == GE_F32 || d == GE_F16 || d == GE_BF16; }

bool known_epilog(int e) {
  return e == GE_EPILOG_NONE || e == GE_EPILOG_RELU_BIAS || e == GE_EPILOG_GELU_BIAS ||
         e == GE_EPILOG_RELU_AUX_BIAS || e == GE_EPILOG_DRELU_BGRAD || e == GE_EPILOG_BIAS ||
         e == GE_EPILOG_RELU_BIAS_UNFUSED;
}

bool uses_bias(ge_epilog_t e) {
  return e == GE_EPILOG_RELU_BIAS || e == GE_EPILOG_GELU_BIAS || e == GE_EPILOG_RELU_AUX_BIAS ||
         e == GE_EPILOG_BIAS || e == GE_EPILOG_RELU_BIAS_UNFUSED;
}

const char* dt_name(ge_dtype_t d) { return d == GE_F32 ? "f32" : d == GE_F16 ? "f16" : "bf16"; }

const char* ep_name(ge_epilog_t e) {
  switch (e) {
    case GE_EPILOG_NONE: return "NONE";
    case GE_EPILOG_RELU_BIAS: return "RELU_BIAS";
    case GE_EPILOG_GELU_BIAS: return "GELU_BIAS";
    case GE_EPILOG_RELU_AUX_BIAS: return "RELU_AUX_BIAS";
    case GE_EPILOG_DRELU_BGRAD: return "DRELU_BGRAD";
    case GE_EPILOG_BIAS: return "BIAS";
    case GE_EPILOG_RELU_BIAS_UNFUSED: return "RELU_BIAS_UNFUSED";
  }
  return "?";
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// An environment switch set to "0" (tuning experiments).
bool env_off(const char* name) {
  const char* v = std::getenv(name);
  return v && v[0] == '0' && v[1] == 0;
}

// 16-bit types, by the number T of 256 x 256 tiles and of 64-wide k-tiles KT
// (measured at 4096x2752x4096, 4096x3200x4096, 8192x1024x8192, 2048x2048x8192,
// 2048x1024x16384, 3072x2560x4096, 4096x1376x4096, 2048^3 and 1024x1024x4096):
//   T >= CUs:      the 256 x 256 tile;
//   T > CUs / 2:   still the 256 x 256 tile, one partly filled round (15-18% faster
//                  than 128 x 128 tiles, which would need more than one round of two
//                  workgroups per CU);
//   KT >= 128:     the 256 x 256 tile with its k loop split across the idle CUs (3-9%
//                  faster: long runs amortise the partial sums); not for transposed
//                  operands, whose plans do not split;
//   otherwise:     the 128 x 128 tile (two workgroups per compute unit), with four
//                  waves of 64 x 64 (LM4) when its grid fills the CUs without a
//                  split and KT >= 64 or two workgroups per CU, else eight waves of
//                  32 x 64 (LM).
// fp32: the register-staged tiles, the largest that still gives every compute unit a
// tile. With an operand stored transposed (lay != 0) the 256 x 256 tile never splits its
// k loop.
int choose_cfg(int64_t m, int n, int64_t k, ge_dtype_t ab, int cus, int lay) {
  const char* env = std::getenv("GE_TILE");
  if (env && env[0]) {
    for (int c = 0; c < gek::CFG_COUNT; ++c)
      if (std::strcmp(env, gek::kTiles[c].name) == 0 && (ab != GE_F32 || !gek::cfg_is_dtl(c)) &&
          (lay == 0 || gek::cfg_has_layouts(c)))
        return c;
  }
  auto tiles = [&](int c) { return cdiv(m, gek::kTiles[c].bm) * cdiv(n, gek::kTiles[c].bn); };
  if (ab != GE_F32) {
    const int64_t t = tiles(gek::CFG_L);
    const int64_t kt = cdiv(k, gek::kTiles[gek::CFG_L].bk);
    if (t >= cus || 2 * t > cus || (kt >= 128 && lay == 0)) return gek::CFG_L;
    // 128 x 128 tiles: four waves of 64 x 64 (LM4) beat eight of 32 x 64 (LM) by 1-2.4%
    // once the grid fills the CUs and either k spans 64 or more k-tiles or the grid
    // fills two workgroups per CU; LM4 cannot split a sparse grid's k loop (measured at
    // 4096x1376x4096, 3072x2560x4096, 2048x2048x4096, 4096x2048x2048, 2048x4096x6144;
    // LM stays ahead at 2048^3 and 1536x2048x4096)
    const int64_t tm = tiles(gek::CFG_LM), rem = tm % (2 * (int64_t)cus);
    const bool lm_splits = rem != 0 && 2 * rem <= cus && kt >= 2;
    if (lay == 0 && !lm_splits && tm >= cus && (kt >= 64 || tm >= 2 * (int64_t)cus)) return gek::CFG_LM4;
    return gek::CFG_LM;
  }
  if (tiles(gek::CFG_M) >= cus) return gek::CFG_M;
  return gek::CFG_S;
}

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
  ge_plan* h = new (std::nothrow) ge_plan();
  if (!h) return GE_ERR_ALLOC;
  h->m = m;
  h->n = (int)n;
  h->k = (int)k;
  h->dt = dt;
  h->ep = ep;
  h->device = dev;
  h->lay = lay;
  h->cus = cus;
  h->cfg = cfg;
  h->allow_split = allow_split;
  h->allow_persist = allow_persist;
  const gek::TileCfg& tc = gek::kTiles[h->cfg];
  h->tiles_m = (int)cdiv(m, tc.bm);
  h->tiles_n = (int)cdiv(n, tc.bn);
  // Tiles that run together on an XCD (32 of them) share A and B in its L2: groups of
  // 8 m-tiles read 8 A and 4 B panels per round. When A outgrows the 256 MB MALL its
  // panels come back from HBM each round, and groups of 4 (4 A and 8 B panels) read
  // 3-4% faster (measured at 16384x16384x8192, 32768x8192x8192 and 65536x8192x16384).
  const double a_bytes = (double)m * (double)k * (double)elem_size(dt.ab);
  h->group_m = a_bytes >= 256.0 * 1024 * 1024 ? 4 : 8;
  if (const char* g = std::getenv("GE_GROUP_M")) {
    const int v = std::atoi(g);
    if (v >= 1 && v <= 1024) h->group_m = v;
  }
  const int kernel_ep = ep == GE_EPILOG_RELU_BIAS_UNFUSED ? (int)gek::NONE : (int)ep;
  h->gemm = lookup(dt.ab, kernel_ep, h->cfg, lay);
  if (!h->gemm) {
    delete h;
    return GE_ERR_NOT_SUPPORTED;
  }

  // ---- split tail: a last round of tiles at most half full shares its K loop ----
  // (split runs start at different k, so they share less of A and B in L2 than whole
  // tiles do and run about 1.4x slower per k-tile: splitting pays when it saves more
  // than that, i.e. when the last round is at most half full)
  const int tiles = h->tiles_m * h->tiles_n;
  h->dp_tiles = tiles;
  if (gek::cfg_can_split(h->cfg) && lay == 0 && allow_split) {
    const int kt = (int)cdiv(k, tc.bk);
    // a round holds one workgroup per CU, two for the 128 x 128 tile (64 KB of LDS): a
    // grid of up to 2 CUs tiles of that size runs in one round and has no sparse tail
    const int slots = h->cfg == gek::CFG_LM ? 2 * cus : cus;
    const int rem = tiles % slots;
    if (rem != 0 && (int64_t)rem * 2 <= (int64_t)cus && kt >= 2) {
      const int64_t units = (int64_t)rem * kt;
      // runs of at least a quarter tile: an owner then adds at most about four partials
      int64_t per = std::max(cdiv(units, cus), cdiv(kt, 4));
      // (experiments: GE_SK_RUN sets the run length, never below one run per compute
      // unit, so every split workgroup is resident at once and every wait ends)
      if (const char* e = std::getenv("GE_SK_RUN")) {
        const int64_t v = std::atoll(e);
        if (v >= 1) per = std::max(v, cdiv(units, cus));
      }
      if (per < kt) {   // a run of k-tiles then holds at most one tile start
        h->dp_tiles = tiles - rem;
        h->sk_units = (int)per;
        h->sk_wgs = (int)cdiv(units, per);
      }
    }
  }

  // ---- persistent kernel: one workgroup per compute unit walks the tiles ----
  if (gek::cfg_can_persist(h->cfg) && h->dp_tiles == tiles && allow_persist) {
    const int kt = (int)cdiv(k, tc.bk);
    if (k % tc.bk == 0 && kt % tc.stages == 0 && kt >= 2 * tc.stages) h->persist_grid = std::min(tiles, cus);
  }

  // ---- workspace: [DRELU_BGRAD row sums | unfused T1, T2][split partials][split flags] ----
  const size_t es = elem_size(dt.d);
  size_t main_bytes = 0;
  if (ep == GE_EPILOG_DRELU_BGRAD) {
    h->partial_cols = (int)cdiv(n, tc.wn);
    main_bytes = (size_t)h->partial_cols * (size_t)m * sizeof(float);
  } else if (ep == GE_EPILOG_RELU_BIAS_UNFUSED) {
    main_bytes = 2 * (size_t)m * (size_t)n * es;
  }
  main_bytes = (main_bytes + 255) & ~(size_t)255;
  const size_t sk_part_bytes = (size_t)h->sk_wgs * gek::sk_slot_bytes(tc);
  const size_t sk_flag_bytes = ((size_t)h->sk_wgs * sizeof(uint32_t) + 255) & ~(size_t)255;
  h->ws_bytes = main_bytes + sk_part_bytes + sk_flag_bytes;
  if (h->ws_bytes) {
    if (hipMalloc(&h->ws, h->ws_bytes) != hipSuccess) {
      delete h;
      return GE_ERR_ALLOC;
    }
    char* base = static_cast<char*>(h->ws);
    if (ep == GE_EPILOG_DRELU_BGRAD) {
      h->partial = reinterpret_cast<float*>(base);
    } else if (ep == GE_EPILOG_RELU_BIAS_UNFUSED) {
      h->t1 = base;
      h->t2 = base + (size_t)m * (size_t)n * es;
    }
    if (h->sk_wgs) {
      h->sk_partial = reinterpret_cast<float*>(base + main_bytes);
      h->sk_flag = reinterpret_cast<uint32_t*>(base + main_bytes + sk_part_bytes);
      // epochs start at 1, so cleared flags never match
      if (hipMemset(h->sk_flag, 0, sk_flag_bytes) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
        hipFree(h->ws);
        delete h;
        return GE_ERR_HIP;
      }
    }
  }
  h->desc = std::string(dt_name(dt.ab)) + " " + ep_name(ep) +
            (lay ? std::string(" op_a ") + (lay & 1 ? "T" : "N") + " op_b " + (lay & 2 ? "T" : "N") : std::string()) +
            " tile " + std::to_string(tc.bm) + "x" +
            std::to_string(tc.bn) + " waves " + std::to_string(tc.bm / tc.wm) + "x" +
            std::to_string(tc.bn / tc.wn) + (gek::cfg_is_dtl(h->cfg) ? " bk " + std::to_string(tc.bk) + " stages " +
                                                 std::to_string(tc.stages) + " " + tc.loop : std::string()) +
            " grid " + std::to_string(h->tiles_m * h->tiles_n) +
            (h->persist_grid ? " on " + std::to_string(h->persist_grid) + " persistent workgroups" : std::string()) +
            (h->sk_wgs ? " (" + std::to_string(h->dp_tiles) + " whole + " + std::to_string(tiles - h->dp_tiles) +
                             " split over " + std::to_string(h->sk_wgs) + "x" + std::to_string(h->sk_units) +
                             " k-tiles)"
                       : std::string());
  if (const char* lg = std::getenv("GE_LOG"); lg && lg[0] == '1')
    std::fprintf(stderr, "gemm_epilog_plan: m=%lld n=%lld k=%lld -> %s, workspace %zu bytes\n", (long long)m,
                 (long long)n, (long long)k, h->desc.c_str(), h->ws_bytes);
  *out = h;
  return GE_OK;
}

}  // namespace

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
  }
  return "unknown status";
}

size_t gemm_epilog_aux_bytes(int64_t m, int64_t n) {
  if (m < 1 || n < 1) return 0;
  return (size_t)4 * (size_t)cdiv(m, 32) * (size_t)n;
}

ge_status_t gemm_epilog_plan(int64_t m, int64_t n, int64_t k, ge_dtypes_t dt, ge_epilog_t ep, ge_handle_t* out) {
  return gemm_epilog_plan_ex(m, n, k, dt, ep, GE_OP_N, GE_OP_N, out);
}

ge_status_t gemm_epilog_plan_ex(int64_t m, int64_t n, int64_t k, ge_dtypes_t dt, ge_epilog_t ep, ge_op_t op_a,
                                ge_op_t op_b, ge_handle_t* out) {
  // ---- host-only validation (no HIP call before this block passes) ----
  if (!out) return GE_ERR_NULL_POINTER;
  if (m < 1 || m > 0x7fffffffLL || n < 1 || n > (1LL << 20) || k < 1 || k > (1LL << 20))
    return GE_ERR_INVALID_VALUE;
  if (!known_dtype(dt.ab) || !known_dtype(dt.d) || !known_dtype(dt.vec) || !known_epilog(ep))
    return GE_ERR_INVALID_VALUE;
  if ((op_a != GE_OP_N && op_a != GE_OP_T) || (op_b != GE_OP_N && op_b != GE_OP_T)) return GE_ERR_INVALID_VALUE;
  if (dt.d != dt.ab) return GE_ERR_NOT_SUPPORTED;
  if (dt.vec != dt.d && dt.vec != GE_F32) return GE_ERR_NOT_SUPPORTED;
  const int64_t mult = dt.ab == GE_F32 ? 4 : 8;   // 16-byte rows
  if (n % mult != 0 || k % mult != 0) return GE_ERR_NOT_SUPPORTED;
  const int lay = (op_a == GE_OP_T ? 1 : 0) | (op_b == GE_OP_T ? 2 : 0);
  if (lay != 0 && dt.ab == GE_F32) return GE_ERR_NOT_SUPPORTED;
  // A stored as (k, m): its rows hold m values, so m follows the row rules of n
  if (op_a == GE_OP_T && (m > (1LL << 20) || m % mult != 0)) return GE_ERR_NOT_SUPPORTED;
  const int64_t tiles_bound = cdiv(m, 64) * cdiv(n, 64);
  if (tiles_bound > 0x7fffffffLL) return GE_ERR_NOT_SUPPORTED;   // grid size

  // ---- device query ----
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return GE_ERR_HIP;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return GE_ERR_HIP;
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return GE_ERR_NOT_SUPPORTED;
  const int cus = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 256;

  return build_plan(m, n, k, dt, ep, lay, dev, cus, choose_cfg(m, (int)n, k, dt.ab, cus, lay), !env_off("GE_STREAMK"),
                    !env_off("GE_PERSIST"), out);
}

ge_status_t gemm_epilog_execute(ge_handle_t h, const void* A, const void* B, const void* bias, void* D, void* aux,
                                void* bgrad, void* stream) {
  // ---- host-only validation ----
  if (!h) return GE_ERR_NULL_POINTER;
  if (!A || !B || !D) return GE_ERR_NULL_POINTER;
  if (!aligned(A, 16) || !aligned(B, 16) || !aligned(D, 16)) return GE_ERR_MISALIGNED;
  const size_t vs = elem_size(h->dt.vec);
  if (uses_bias(h->ep)) {
    if (!bias) return GE_ERR_NULL_POINTER;
    if (!aligned(bias, vs)) return GE_ERR_MISALIGNED;
  }
  if (h->ep == GE_EPILOG_RELU_AUX_BIAS || h->ep == GE_EPILOG_DRELU_BGRAD) {
    if (!aux) return GE_ERR_NULL_POINTER;
    if (!aligned(aux, 16)) return GE_ERR_MISALIGNED;
  }
  if (h->ep == GE_EPILOG_DRELU_BGRAD) {
    if (!bgrad) return GE_ERR_NULL_POINTER;
    if (!aligned(bgrad, vs)) return GE_ERR_MISALIGNED;
  }

  hipStream_t s = static_cast<hipStream_t>(stream);
  gek::Args a;
  a.A = A;
  a.B = B;
  a.bias = bias;
  a.D = (h->ep == GE_EPILOG_RELU_BIAS_UNFUSED) ? h->t1 : D;
  a.aux = static_cast<uint32_t*>(aux);
  a.partial = h->partial;
  a.m = h->m;
  a.n = h->n;
  a.k = h->k;
  a.vec_dt = (int)h->dt.vec;
  a.tiles_m = h->tiles_m;
  a.tiles_n = h->tiles_n;
  a.group_m = h->group_m;
  a.dp_tiles = h->dp_tiles;
  a.sk_units = h->sk_units;
  a.sk_wgs = h->sk_wgs;
  a.sk_partial = h->sk_partial;
  a.sk_flag = h->sk_flag;
  a.persist_grid = h->persist_grid;
  h->epoch = h->epoch % 0x7fffffffu + 1u;
  a.epoch = h->epoch;
  const int grid = h->tiles_m * h->tiles_n;

  if (h->gemm(a, grid, s) != hipSuccess) return GE_ERR_HIP;
  if (h->ep == GE_EPILOG_DRELU_BGRAD) {
    if (gek::launch_bgrad_reduce(h->partial, h->partial_cols, h->m, bgrad, (int)h->dt.vec, s) != hipSuccess)
      return GE_ERR_HIP;
  } else if (h->ep == GE_EPILOG_RELU_BIAS_UNFUSED) {
    if (gek::launch_bias_add((int)h->dt.d, h->t1, bias, (int)h->dt.vec, h->t2, h->m, h->n, s) != hipSuccess)
      return GE_ERR_HIP;
    if (gek::launch_relu((int)h->dt.d, h->t2, D, h->m, h->n, s) != hipSuccess) return GE_ERR_HIP;
  }
  return GE_OK;
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
  } else if (h->lay != 0) {
    cands = {{gek::CFG_L, false, true}, {gek::CFG_L, false, false}, {gek::CFG_LH, false, false},
             {gek::CFG_LM, false, false}};
  } else {
    cands = {{gek::CFG_L, true, true},   {gek::CFG_L, false, true},   {gek::CFG_L, false, false},
             {gek::CFG_LH, true, false}, {gek::CFG_LH, false, false}, {gek::CFG_LM, true, false},
             {gek::CFG_LM, false, false}, {gek::CFG_LM4, false, false}};
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
    if (build_plan(h->m, h->n, h->k, h->dt, h->ep, h->lay, h->device, h->cus, c.cfg, c.split, c.persist, &t) !=
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

ge_status_t gemm_epilog_free(ge_handle_t h) {
  if (!h) return GE_OK;
  ge_status_t st = GE_OK;
  if (h->ws && hipFree(h->ws) != hipSuccess) st = GE_ERR_HIP;
  delete h;
  return st;
}

size_t gemm_epilog_workspace_bytes(ge_handle_t h) { return h ? h->ws_bytes : 0; }

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
  const dim3 grid((unsigned)cdiv(chunks, 256));
  void* params[] = {&in, &bias, &vec_dt, &out, const_cast<int64_t*>(&chunks), &n};
  const void* fn = dt == F32 ? reinterpret_cast<const void*>(&bias_add_kernel<F32>)
                 : dt == F16 ? reinterpret_cast<const void*>(&bias_add_kernel<F16>)
                             : reinterpret_cast<const void*>(&bias_add_kernel<BF16>);
  return hipLaunchKernel(fn, grid, dim3(256), params, 0, s);
}

hipError_t launch_relu(int dt, const void* in, void* out, int64_t m, int n, hipStream_t s) {
  const int E = dt == F32 ? 4 : 8;
  const int64_t chunks = m * (int64_t)n / E;
  const dim3 grid((unsigned)cdiv(chunks, 256));
  void* params[] = {&in, &out, const_cast<int64_t*>(&chunks)};
  const void* fn = dt == F32 ? reinterpret_cast<const void*>(&relu_kernel<F32>)
                 : dt == F16 ? reinterpret_cast<const void*>(&relu_kernel<F16>)
                             : reinterpret_cast<const void*>(&relu_kernel<BF16>);
  return hipLaunchKernel(fn, grid, dim3(256), params, 0, s);
}

hipError_t launch_bgrad_reduce(const float* partial, int t, int64_t m, void* bgrad, int vec_dt, hipStream_t s) {
  const dim3 grid((unsigned)cdiv(m, 64));
  void* params[] = {&partial, &t, &m, &bgrad, &vec_dt};
  return hipLaunchKernel(reinterpret_cast<const void*>(&bgrad_reduce_kernel), grid, dim3(64 * kReduceWaves), params,
                         0, s);
}

}  // namespace gek
