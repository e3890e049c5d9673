// Host-side plan arithmetic (declared in plan_host.hpp): no HIP call, builds with g++.
//
// The plan step follows "nvmath-python wraps cuBLASLt" (blog.hotdry.top), body: the
// costly choices are made once when planning, execution is light and repeated; the
// argument rules follow "Fusing bias addition via the nvmath-python epilog mechanism"
// (blog.hotdry.top), paragraph 4, first item: the bias type must agree with the
// matrices (the same 16-bit type, or fp32).

#include "plan_host.hpp"

#include <algorithm>
#include <cstdlib>
#include <cstring>

#include "tiles.hpp"

static_assert(geh::kSkFlagRegion == gek::kSkFlagWords * sizeof(uint32_t), "flag region");

namespace geh {

namespace {

bool known_dtype(int d) { return d == GE_F32 || d == GE_F16 || d == GE_BF16; }

bool known_epilog(int e) {
  return e == GE_EPILOG_NONE || e == GE_EPILOG_RELU_BIAS || e == GE_EPILOG_GELU_BIAS ||
         e == GE_EPILOG_RELU_AUX_BIAS || e == GE_EPILOG_DRELU_BGRAD || e == GE_EPILOG_BIAS ||
         e == GE_EPILOG_RELU_BIAS_UNFUSED || e == GE_EPILOG_DRELU_BGRAD_UNFUSED;
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
    case GE_EPILOG_DRELU_BGRAD_UNFUSED: return "DRELU_BGRAD_UNFUSED";
  }
  return "?";
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

}  // namespace

size_t elem_size(ge_dtype_t d) { return d == GE_F32 ? 4 : 2; }

bool uses_bias(ge_epilog_t e) {
  return e == GE_EPILOG_RELU_BIAS || e == GE_EPILOG_GELU_BIAS || e == GE_EPILOG_RELU_AUX_BIAS ||
         e == GE_EPILOG_BIAS || e == GE_EPILOG_RELU_BIAS_UNFUSED;
}

int64_t split_run_length(int64_t rem, int64_t kt, int cus) {
  // one run per CU at most, and runs of at least a quarter tile: an owner then adds at
  // most about four partials
  return std::max(cdiv(rem * kt, cus), cdiv(kt, 4));
}

bool is_unfused(ge_epilog_t e) { return e == GE_EPILOG_RELU_BIAS_UNFUSED || e == GE_EPILOG_DRELU_BGRAD_UNFUSED; }

int gemm_epilog_of(ge_epilog_t e) { return is_unfused(e) ? (int)GE_EPILOG_NONE : (int)e; }

bool env_off(const char* name) {
  const char* v = std::getenv(name);
  return v && v[0] == '0' && v[1] == 0;
}

ge_status_t check_plan_args(int64_t m, int64_t n, int64_t k, ge_dtypes_t dt, ge_epilog_t ep, ge_op_t op_a,
                            ge_op_t op_b, int* lay) {
  if (m < 1 || m > 0x7fffffffLL || n < 1 || n > (1LL << 20) || k < 1 || k > (1LL << 20))
    return GE_ERR_INVALID_VALUE;
  if (!known_dtype(dt.ab) || !known_dtype(dt.d) || !known_dtype(dt.vec) || !known_epilog(ep))
    return GE_ERR_INVALID_VALUE;
  if ((op_a != GE_OP_N && op_a != GE_OP_T) || (op_b != GE_OP_N && op_b != GE_OP_T)) return GE_ERR_INVALID_VALUE;
  if (dt.d != dt.ab) return GE_ERR_NOT_SUPPORTED;
  if (dt.vec != dt.d && dt.vec != GE_F32) return GE_ERR_NOT_SUPPORTED;
  const int64_t mult = dt.ab == GE_F32 ? 4 : 8;   // 16-byte rows
  if (n % mult != 0 || k % mult != 0) return GE_ERR_NOT_SUPPORTED;
  const int l = (op_a == GE_OP_T ? 1 : 0) | (op_b == GE_OP_T ? 2 : 0);
  if (l != 0 && dt.ab == GE_F32) return GE_ERR_NOT_SUPPORTED;
  // A stored as (k, m): its rows hold m values, so m follows the row rules of n
  if (op_a == GE_OP_T && (m > (1LL << 20) || m % mult != 0)) return GE_ERR_NOT_SUPPORTED;
  if (cdiv(m, 64) * cdiv(n, 64) > 0x7fffffffLL) return GE_ERR_NOT_SUPPORTED;   // grid size
  *lay = l;
  return GE_OK;
}

// 16-bit types, by the number T of 256 x 256 tiles, the number TM of 128 x 128 tiles
// and of 64-wide k-tiles KT (measured at 4096x2752x4096, 4096x3200x4096,
// 8192x1024x8192, 2048x2048x8192, 2048x1024x16384, 3072x2560x4096, 4096x1376x4096,
// 2048^3 and 1024x1024x4096, and for LMD at 26 shapes from 1024x512x2048 to
// 2048x2048x16384, fp16 and bf16, forward and backward, A or B transposed):
//   T >= CUs:      the 256 x 256 tile;
//   T > CUs / 2:   still the 256 x 256 tile, one partly filled round (15-18% faster
//                  than 128 x 128 tiles, which would need more than one round of two
//                  workgroups per CU);
//                  in both cases the 192 x 256 tile (L3) instead when its T3 tiles take
//                  no more rounds than T, are more (a fuller last round) and leave no
//                  last round to split: 0.3-8.8% faster at 4096x2752x4096,
//                  3072x4096x4096, 6144x4096x4096, 8448x4096x4096 and seven more shapes.
//                  It loses where it needs more rounds (8192^3 11%, 4096^3 27%), where
//                  both fill whole rounds (2-3% per flop), and where its last round is
//                  split into runs that do not divide the k loop (4352x4096x4096: 9-13%).
//                  The power limit keeps the gain below the CUs' share: a round that
//                  leaves CUs idle runs at a higher clock;
//   TM <= CUs:     the 128 x 128 tile with a 3-stage ring (LMD, 96 KB: one workgroup
//                  per CU, which such a grid has anyway) when each workgroup's k loop is
//                  long enough for the ring to hide the copies' latency: split runs of
//                  12 to 64 k-tiles (5-16% faster than the 2-stage ring; 3-51% faster
//                  than the 256 x 256 split at KT >= 128, which stays 4% ahead with runs
//                  of 128), or whole tiles of 24 to 127 k-tiles (3-20% faster; at 16-20
//                  k-tiles it is 1-2% slower, and from 128 on the 256 x 256 split stays
//                  7% ahead);
//   KT >= 128:     the 256 x 256 tile with its k loop split across the idle CUs (3-9%
//                  faster than the 2-stage 128 x 128 tile: long runs amortise the partial
//                  sums; 1-7% faster than the 128 x 256 tile at 2048x4096x8192,
//                  4096x2048x8192 and 2048x4096x16384); not for transposed operands,
//                  whose plans do not split;
//   TW in (CUs / 2, CUs], TW the 128 x 256 tiles, n padded by at most 5%: the
//                  persistent 128 x 256 tile (LW; eight waves of 64 x 64, one
//                  workgroup per CU) where two 128 x 128 workgroups per CU would run:
//                  1.3-7.5% faster at 4096x2048x2048, 4096x2048x4096, 2048x4096x4096,
//                  2048x4096x6144, 2048x3072x4096, 1536x4096x4096 and 3072x2560x4096 (it
//                  copies 25% fewer bytes per flop); 3-6% slower at 4096x1376x4096,
//                  whose n pads to 1536;
//   otherwise:     the 128 x 128 tile (two workgroups per compute unit), with four
//                  waves of 64 x 64 (LM4) when its grid fills the CUs without a
//                  split and KT >= 64 or two workgroups per CU, else eight waves of
//                  32 x 64 (LM).
// fp32: the register-staged tiles, the largest that still gives every compute unit a
// tile. With an operand stored transposed (lay != 0) the 256 x 256 tile never splits its
// k loop.
int choose_cfg(int64_t m, int64_t n, int64_t k, ge_dtype_t ab, int cus, int lay) {
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
    if (t >= cus || 2 * t > cus) {
      const int64_t t3 = tiles(gek::CFG_L3);
      const int64_t rem3 = t3 % cus;
      if (lay == 0 && t3 > t && cdiv(t3, cus) <= cdiv(t, cus) && (rem3 == 0 || 2 * rem3 > cus))
        return gek::CFG_L3;
      return gek::CFG_L;
    }
    const int64_t tm = tiles(gek::CFG_LM);
    if (tm <= cus) {
      if (lay == 0 && 2 * tm <= cus && kt >= 2) {   // LMD splits this grid's k loops
        const int64_t run = split_run_length(tm, kt, cus);
        if (run >= 12 && run <= 64) return gek::CFG_LMD;
      } else if (kt >= 24 && (kt < 128 || lay != 0)) {
        return gek::CFG_LMD;
      }
    }
    if (kt >= 128 && lay == 0) return gek::CFG_L;
    if (lay == 0) {
      const int64_t tw = tiles(gek::CFG_LW), npad = cdiv(n, 256) * 256;
      if (2 * tw > cus && tw <= cus && 20 * (npad - n) <= npad) return gek::CFG_LW;
    }
    // 128 x 128 tiles: four waves of 64 x 64 (LM4) beat eight of 32 x 64 (LM) by 1-2.4%
    // once the grid fills the CUs and either k spans 64 or more k-tiles or the grid
    // fills two workgroups per CU; LM4 cannot split a sparse grid's k loop (measured at
    // 4096x1376x4096, 3072x2560x4096, 2048x2048x4096, 4096x2048x2048, 2048x4096x6144;
    // LM stays ahead at 2048^3 and 1536x2048x4096)
    const int64_t rem = tm % (2 * (int64_t)cus);
    const bool lm_splits = rem != 0 && 2 * rem <= cus && kt >= 2;
    if (lay == 0 && !lm_splits && tm >= cus && (kt >= 64 || tm >= 2 * (int64_t)cus)) return gek::CFG_LM4;
    return gek::CFG_LM;
  }
  if (tiles(gek::CFG_M) >= cus) return gek::CFG_M;
  return gek::CFG_S;
}

ge_status_t make_layout(int64_t m, int64_t n, int64_t k, ge_dtypes_t dt, ge_epilog_t ep, int lay, int cus, int cfg,
                        bool allow_split, bool allow_persist, Layout* out) {
  if (cfg < 0 || cfg >= gek::CFG_COUNT || cus < 1) return GE_ERR_INVALID_VALUE;
  if (dt.ab == GE_F32 && gek::cfg_is_dtl(cfg)) return GE_ERR_NOT_SUPPORTED;
  if (lay != 0 && !gek::cfg_has_layouts(cfg)) return GE_ERR_NOT_SUPPORTED;
  Layout L;
  L.cfg = cfg;
  L.lay = lay;
  const gek::TileCfg& tc = gek::kTiles[cfg];
  L.tiles_m = (int)cdiv(m, tc.bm);
  L.tiles_n = (int)cdiv(n, tc.bn);
  // Tiles that run together on an XCD (32 of them) share A and B in its L2: groups of
  // 8 m-tiles read 8 A and 4 B panels per round. When A outgrows the 256 MB MALL its
  // panels come back from HBM each round, and groups of 4 (4 A and 8 B panels) read
  // 3-4% faster (measured at 16384x16384x8192, 32768x8192x8192 and 65536x8192x16384).
  const double a_bytes = (double)m * (double)k * (double)elem_size(dt.ab);
  L.group_m = a_bytes >= 256.0 * 1024 * 1024 ? 4 : 8;

  // ---- split tail: a last round of tiles at most half full shares its K loop ----
  // (split runs start at different k, so they share less of A and B in L2 than whole
  // tiles do and run about 1.4x slower per k-tile: splitting pays when it saves more
  // than that, i.e. when the last round is at most half full)
  const int64_t tiles = (int64_t)L.tiles_m * L.tiles_n;
  L.dp_tiles = (int)tiles;
  if (gek::cfg_can_split(cfg) && lay == 0 && allow_split) {
    const int64_t kt = cdiv(k, tc.bk);
    // a round holds one workgroup per CU, two for the 2-stage 128 x 128 tile (64 KB of LDS): a
    // grid of up to 2 CUs tiles of that size runs in one round and has no sparse tail
    const int64_t slots = cfg == gek::CFG_LM ? 2 * (int64_t)cus : cus;
    const int64_t rem = tiles % slots;
    if (rem != 0 && rem * 2 <= (int64_t)cus && kt >= 2) {
      const int64_t units = rem * kt;
      int64_t per = split_run_length(rem, kt, cus);
      // (experiments: GE_SK_RUN sets the run length, never below one run per compute
      // unit, so every split workgroup is resident at once and every wait ends)
      if (const char* e = std::getenv("GE_SK_RUN")) {
        const int64_t v = std::atoll(e);
        if (v >= 1) per = std::max(v, cdiv(units, cus));
      }
      // a run of k-tiles holds at most one tile start when per < kt; every split
      // workgroup's flag fits the fixed flag region
      if (per < kt && cdiv(units, per) < (int64_t)gek::kSkLostWord) {
        L.dp_tiles = (int)(tiles - rem);
        L.sk_units = (int)per;
        L.sk_wgs = (int)cdiv(units, per);
        L.sk_parts = kt % per == 0 ? (int)(kt / per) : 0;
      }
    }
  }

  // Split runs of one XCD cover fewer tiles, each over part of its k loop: groups of 4
  // m-tiles give those tiles fewer distinct A and B panels (1024x1024x4096: 20.7 against
  // 21.8 us with groups of 8; the split 256 x 256 shapes 0.2-0.5% faster).
  if (L.sk_wgs > 0) L.group_m = 4;
  if (const char* g = std::getenv("GE_GROUP_M")) {
    const int v = std::atoi(g);
    if (v >= 1 && v <= 1024) L.group_m = v;
  }

  // ---- persistent kernel: one workgroup per compute unit walks the tiles ----
  if (gek::cfg_can_persist(cfg) && L.dp_tiles == tiles && allow_persist) {
    const int64_t kt = cdiv(k, tc.bk);
    if (k % tc.bk == 0 && kt % tc.stages == 0 && kt >= 2 * tc.stages) L.persist_grid = (int)std::min<int64_t>(tiles, cus);
  }

  // ---- workspace: [split flags][DRELU_BGRAD row sums | unfused T1 (and T2)][split partials] ----
  // The flags (one word per split workgroup, and the count of owner waits that ran out
  // in the region's last word) come first, in a region of fixed size, so their place
  // does not move with the problem: a workspace reused across problems keeps them at 0
  // between executes.
  const size_t es = elem_size(dt.d);
  L.sk_flag_bytes = L.sk_wgs ? kSkFlagRegion : 0;
  L.off_sk_flag = 0;
  const size_t main_off = L.sk_flag_bytes;
  size_t main_bytes = 0;
  if (ep == GE_EPILOG_DRELU_BGRAD) {
    L.partial_cols = (int)cdiv(n, tc.wn);
    main_bytes = (size_t)L.partial_cols * (size_t)m * sizeof(float);
    L.off_partial = main_off;
  } else if (ep == GE_EPILOG_RELU_BIAS_UNFUSED) {
    main_bytes = 2 * (size_t)m * (size_t)n * es;
    L.off_t1 = main_off;
    L.off_t2 = main_off + (size_t)m * (size_t)n * es;
  } else if (ep == GE_EPILOG_DRELU_BGRAD_UNFUSED) {
    main_bytes = (size_t)m * (size_t)n * es;
    L.off_t1 = main_off;
  }
  L.off_sk_partial = main_off + align256(main_bytes);
  L.ws_bytes = L.off_sk_partial + (size_t)L.sk_wgs * gek::sk_slot_bytes(tc);
  *out = L;
  return GE_OK;
}

std::string describe(ge_dtypes_t dt, ge_epilog_t ep, const Layout& L) {
  const gek::TileCfg& tc = gek::kTiles[L.cfg];
  const int tiles = L.tiles_m * L.tiles_n;
  std::string s = std::string(dt_name(dt.ab)) + " " + ep_name(ep);
  if (L.lay) s += std::string(" op_a ") + (L.lay & 1 ? "T" : "N") + " op_b " + (L.lay & 2 ? "T" : "N");
  s += " tile " + std::to_string(tc.bm) + "x" + std::to_string(tc.bn) + " waves " + std::to_string(tc.bm / tc.wm) +
       "x" + std::to_string(tc.bn / tc.wn);
  if (gek::cfg_is_dtl(L.cfg))
    s += " bk " + std::to_string(tc.bk) + " stages " + std::to_string(tc.stages) + " " + tc.loop;
  s += " grid " + std::to_string(tiles);
  if (L.persist_grid) s += " on " + std::to_string(L.persist_grid) + " persistent workgroups";
  if (L.sk_wgs)
    s += " (" + std::to_string(L.dp_tiles) + " whole + " + std::to_string(tiles - L.dp_tiles) + " split over " +
         std::to_string(L.sk_wgs) + "x" + std::to_string(L.sk_units) + " k-tiles" +
         (L.sk_parts ? ", " + std::to_string(L.sk_parts) + " parts per tile)" : ")");
  return s;
}

ge_status_t check_execute_args(ge_epilog_t ep, ge_dtypes_t dt, const void* A, const void* B, const void* bias,
                               const void* D, const void* aux, const void* bgrad) {
  if (!A || !B || !D) return GE_ERR_NULL_POINTER;
  if (!aligned(A, 16) || !aligned(B, 16) || !aligned(D, 16)) return GE_ERR_MISALIGNED;
  const size_t vs = elem_size(dt.vec);
  if (uses_bias(ep)) {
    if (!bias) return GE_ERR_NULL_POINTER;
    if (!aligned(bias, vs)) return GE_ERR_MISALIGNED;
  }
  if (ep == GE_EPILOG_RELU_AUX_BIAS || ep == GE_EPILOG_DRELU_BGRAD || ep == GE_EPILOG_DRELU_BGRAD_UNFUSED) {
    if (!aux) return GE_ERR_NULL_POINTER;
    if (!aligned(aux, 16)) return GE_ERR_MISALIGNED;
  }
  if (ep == GE_EPILOG_DRELU_BGRAD || ep == GE_EPILOG_DRELU_BGRAD_UNFUSED) {
    if (!bgrad) return GE_ERR_NULL_POINTER;
    if (!aligned(bgrad, vs)) return GE_ERR_MISALIGNED;
  }
  return GE_OK;
}

}  // namespace geh

extern "C" ge_status_t gemm_epilog_plan_info(int64_t m, int64_t n, int64_t k, ge_dtypes_t dt, ge_epilog_t ep,
                                             ge_op_t op_a, ge_op_t op_b, int compute_units, ge_plan_info_t* info) {
  if (!info) return GE_ERR_NULL_POINTER;
  if (compute_units < 1 || compute_units > 4096) return GE_ERR_INVALID_VALUE;
  int lay = 0;
  if (ge_status_t st = geh::check_plan_args(m, n, k, dt, ep, op_a, op_b, &lay); st != GE_OK) return st;
  geh::Layout L;
  const int cfg = geh::choose_cfg(m, n, k, dt.ab, compute_units, lay);
  if (ge_status_t st = geh::make_layout(m, n, k, dt, ep, lay, compute_units, cfg, !geh::env_off("GE_STREAMK"),
                                        !geh::env_off("GE_PERSIST"), &L);
      st != GE_OK)
    return st;
  const gek::TileCfg& tc = gek::kTiles[cfg];
  ge_plan_info_t r;
  std::memset(&r, 0, sizeof(r));
  r.tile_m = tc.bm;
  r.tile_n = tc.bn;
  r.tile_k = tc.bk;
  r.waves = (tc.bm / tc.wm) * (tc.bn / tc.wn);
  r.tiles = (int64_t)L.tiles_m * L.tiles_n;
  r.persistent_workgroups = L.persist_grid;
  r.whole_tiles = L.dp_tiles;
  r.split_workgroups = L.sk_wgs;
  r.split_run_ktiles = L.sk_units;
  r.group_m = L.group_m;
  r.workspace_bytes = L.ws_bytes;
  r.stages = gek::cfg_is_dtl(cfg) ? tc.stages : 0;
  *info = r;
  return GE_OK;
}
