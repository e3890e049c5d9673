// Exercises the host plan arithmetic of the library (plan_host.cpp and the constexpr
// tile table / split-run arithmetic of tiles.hpp that the kernels also use) under
// AddressSanitizer and UndefinedBehaviorSanitizer: built by tests/test_plan_sanitize.py
// with g++, host code only. Checks, over a grid of problems:
//   * argument rules: the status codes of invalid sizes, types, storage orders;
//   * layouts: workspace regions 256-byte aligned, inside ws_bytes and disjoint;
//     the tile grid covers the output; the persistent grid only where it applies;
//   * the split tail through gek::sk_run: every (tail tile, k-tile) computed exactly
//     once, one owner piece per tile starting at k = 0, partials never at k = 0 and
//     before the owner piece of their run, the runs an owner waits for are exactly the
//     runs holding the rest of its tile, every split workgroup resident at once.
// Prints "ok (0 failures)" on success.
#include <cstdio>
#include <cstdlib>
#include <set>
#include <utility>
#include <vector>

#include "plan_host.hpp"
#include "tiles.hpp"

namespace {

int failures = 0;

void check(bool ok, const char* what, long long m, long long n, long long k, int cfg) {
  if (!ok) {
    if (failures < 50) std::printf("FAIL %s m=%lld n=%lld k=%lld cfg=%d\n", what, m, n, k, cfg);
    ++failures;
  }
}

ge_dtypes_t dts(ge_dtype_t t) { return ge_dtypes_t{t, t, t}; }

void check_args() {
  int lay = -1;
  const ge_dtypes_t f16 = dts(GE_F16);
  struct Case {
    long long m, n, k;
    ge_dtypes_t dt;
    int ep, oa, ob;
    ge_status_t want;
  } cases[] = {
      {0, 8, 8, f16, GE_EPILOG_RELU_BIAS, 0, 0, GE_ERR_INVALID_VALUE},
      {8, 0, 8, f16, GE_EPILOG_RELU_BIAS, 0, 0, GE_ERR_INVALID_VALUE},
      {8, 8, 0, f16, GE_EPILOG_RELU_BIAS, 0, 0, GE_ERR_INVALID_VALUE},
      {1LL << 31, 8, 8, f16, GE_EPILOG_RELU_BIAS, 0, 0, GE_ERR_INVALID_VALUE},
      {8, (1 << 20) + 8, 8, f16, GE_EPILOG_RELU_BIAS, 0, 0, GE_ERR_INVALID_VALUE},
      {8, 8, 8, f16, 7, 0, 0, GE_ERR_INVALID_VALUE},
      {8, 8, 8, ge_dtypes_t{(ge_dtype_t)3, GE_F16, GE_F16}, GE_EPILOG_RELU_BIAS, 0, 0, GE_ERR_INVALID_VALUE},
      {8, 8, 8, f16, GE_EPILOG_RELU_BIAS, 2, 0, GE_ERR_INVALID_VALUE},
      {8, 8, 8, ge_dtypes_t{GE_F16, GE_BF16, GE_F16}, GE_EPILOG_RELU_BIAS, 0, 0, GE_ERR_NOT_SUPPORTED},
      {8, 8, 8, ge_dtypes_t{GE_F16, GE_F16, GE_BF16}, GE_EPILOG_RELU_BIAS, 0, 0, GE_ERR_NOT_SUPPORTED},
      {8, 12, 8, f16, GE_EPILOG_RELU_BIAS, 0, 0, GE_ERR_NOT_SUPPORTED},
      {8, 8, 12, f16, GE_EPILOG_RELU_BIAS, 0, 0, GE_ERR_NOT_SUPPORTED},
      {12, 8, 8, f16, GE_EPILOG_RELU_BIAS, 1, 0, GE_ERR_NOT_SUPPORTED},
      {8, 8, 8, dts(GE_F32), GE_EPILOG_RELU_BIAS, 0, 1, GE_ERR_NOT_SUPPORTED},
      {12, 8, 8, f16, GE_EPILOG_RELU_BIAS, 0, 1, GE_OK},
      {33, 8, 8, ge_dtypes_t{GE_BF16, GE_BF16, GE_F32}, GE_EPILOG_DRELU_BGRAD, 0, 0, GE_OK},
      {33, 8, 8, ge_dtypes_t{GE_BF16, GE_BF16, GE_F32}, GE_EPILOG_DRELU_BGRAD_UNFUSED, 1, 0, GE_ERR_NOT_SUPPORTED},
      {40, 8, 8, f16, GE_EPILOG_DRELU_BGRAD_UNFUSED, 1, 0, GE_OK},
      {8, 8, 8, f16, 102, 0, 0, GE_ERR_INVALID_VALUE},
  };
  for (const Case& c : cases) {
    const ge_status_t st =
        geh::check_plan_args(c.m, c.n, c.k, c.dt, (ge_epilog_t)c.ep, (ge_op_t)c.oa, (ge_op_t)c.ob, &lay);
    check(st == c.want, "argument rule", c.m, c.n, c.k, -1);
  }
  // execute pointer rules
  alignas(16) static char buf[256];
  const void* p = buf;
  check(geh::check_execute_args(GE_EPILOG_RELU_BIAS, f16, p, p, p, p, nullptr, nullptr) == GE_OK, "exec ok", 0, 0, 0, -1);
  check(geh::check_execute_args(GE_EPILOG_RELU_BIAS, f16, p, p, nullptr, p, nullptr, nullptr) == GE_ERR_NULL_POINTER,
        "exec bias null", 0, 0, 0, -1);
  check(geh::check_execute_args(GE_EPILOG_RELU_BIAS, f16, buf + 2, p, p, p, nullptr, nullptr) == GE_ERR_MISALIGNED,
        "exec A misaligned", 0, 0, 0, -1);
  check(geh::check_execute_args(GE_EPILOG_RELU_AUX_BIAS, f16, p, p, p, p, buf + 4, nullptr) == GE_ERR_MISALIGNED,
        "exec aux misaligned", 0, 0, 0, -1);
  check(geh::check_execute_args(GE_EPILOG_DRELU_BGRAD, f16, p, p, nullptr, p, p, nullptr) == GE_ERR_NULL_POINTER,
        "exec bgrad null", 0, 0, 0, -1);
  check(geh::check_execute_args(GE_EPILOG_DRELU_BGRAD, dts(GE_F32), p, p, nullptr, p, p, buf + 2) ==
            GE_ERR_MISALIGNED,
        "exec bgrad misaligned", 0, 0, 0, -1);
  check(geh::check_execute_args(GE_EPILOG_DRELU_BGRAD_UNFUSED, f16, p, p, nullptr, p, nullptr, p) ==
            GE_ERR_NULL_POINTER,
        "exec unfused backward activation null", 0, 0, 0, -1);
  check(geh::check_execute_args(GE_EPILOG_DRELU_BGRAD_UNFUSED, f16, p, p, nullptr, p, buf + 8, p) == GE_ERR_MISALIGNED,
        "exec unfused backward activation misaligned", 0, 0, 0, -1);
  check(geh::check_execute_args(GE_EPILOG_DRELU_BGRAD_UNFUSED, f16, p, p, nullptr, p, p, nullptr) ==
            GE_ERR_NULL_POINTER,
        "exec unfused backward bgrad null", 0, 0, 0, -1);
  check(geh::check_execute_args(GE_EPILOG_DRELU_BGRAD_UNFUSED, f16, p, p, nullptr, p, p, p) == GE_OK,
        "exec unfused backward ok without a bias", 0, 0, 0, -1);
}

// The split tail of layout L for K k-tiles, through the kernel's own run arithmetic.
void check_split(const geh::Layout& L, int kt, int cus, long long m, long long n, long long k) {
  const int tiles = L.tiles_m * L.tiles_n;
  const int tail = tiles - L.dp_tiles;
  const int total = tail * kt;
  check(L.sk_units >= 1 && L.sk_units < kt, "run shorter than a tile", m, n, k, L.cfg);
  check(L.sk_wgs <= cus, "split workgroups resident at once", m, n, k, L.cfg);
  check((long long)L.sk_wgs * L.sk_units >= total && (long long)(L.sk_wgs - 1) * L.sk_units < total,
        "runs cover the tail exactly", m, n, k, L.cfg);
  std::vector<int> cover((size_t)total, 0);
  std::vector<int> owner((size_t)tail, -1);
  std::vector<int> partial_tile((size_t)L.sk_wgs, -1);
  for (int r = 0; r < L.sk_wgs; ++r) {
    const gek::SkRun s = gek::sk_run(r, L.sk_units, kt, tail, L.sk_wgs);
    if (s.pa_nt > 0) {
      check(s.pa_kb > 0 && s.pa_kb + s.pa_nt <= kt, "partial inside its tile, not at k = 0", m, n, k, L.cfg);
      for (int u = 0; u < s.pa_nt; ++u) ++cover[(size_t)(s.pa_t * kt + s.pa_kb + u)];
      partial_tile[(size_t)r] = s.pa_t;
    }
    if (s.own_nt > 0) {
      check(s.own_t < tail && s.own_nt <= kt, "owner piece inside its tile", m, n, k, L.cfg);
      check(owner[(size_t)s.own_t] < 0, "one owner per tile", m, n, k, L.cfg);
      owner[(size_t)s.own_t] = r;
      for (int u = 0; u < s.own_nt; ++u) ++cover[(size_t)(s.own_t * kt + u)];
      check(s.last >= r && s.last < L.sk_wgs, "owner's last partner in range", m, n, k, L.cfg);
    }
  }
  for (int u = 0; u < total; ++u) check(cover[(size_t)u] == 1, "each k-tile exactly once", m, n, k, L.cfg);
  std::vector<int> waited((size_t)L.sk_wgs, 0);
  for (int t = 0; t < tail; ++t) {
    const int r = owner[(size_t)t];
    check(r >= 0, "every tail tile has an owner", m, n, k, L.cfg);
    if (r < 0) continue;
    const gek::SkRun s = gek::sk_run(r, L.sk_units, kt, tail, L.sk_wgs);
    for (int o = r + 1; o <= s.last; ++o) {
      check(partial_tile[(size_t)o] == t, "a partner holds a partial of the owner's tile", m, n, k, L.cfg);
      ++waited[(size_t)o];
    }
  }
  for (int r = 0; r < L.sk_wgs; ++r)
    check(waited[(size_t)r] == (partial_tile[(size_t)r] >= 0 ? 1 : 0), "each published partial has one waiter", m, n,
          k, L.cfg);
  // runs that cover whole tiles: the kernel takes run r as part r % S of tail tile r / S
  // and counts each tile's publications in flag words 2t and 2t + 1
  check((L.sk_parts != 0) == (kt % L.sk_units == 0), "parts exactly when runs divide the tile", m, n, k, L.cfg);
  if (L.sk_parts) {
    const int S = L.sk_parts;
    check(S >= 2 && S * L.sk_units == kt && L.sk_wgs == tail * S, "parts cover each tile", m, n, k, L.cfg);
    check(2 * tail <= gek::kSkLostWord, "tile counters below the lost-wait word", m, n, k, L.cfg);
    for (int r = 0; r < L.sk_wgs; ++r) {
      const gek::SkRun s = gek::sk_run(r, L.sk_units, kt, tail, L.sk_wgs);
      const int t = r / S, part = r % S;
      if (part == 0)
        check(s.pa_nt == 0 && s.own_t == t && s.own_nt == L.sk_units, "part 0 starts its tile", m, n, k, L.cfg);
      else
        check(s.own_nt == 0 && s.pa_t == t && s.pa_kb == part * L.sk_units && s.pa_nt == L.sk_units,
              "part s covers k-tiles [s units, (s + 1) units)", m, n, k, L.cfg);
    }
  }
}

void check_layout(long long m, long long n, long long k, ge_dtype_t t, ge_epilog_t ep, int cus) {
  const ge_dtypes_t dt = dts(t);
  int lay = 0;
  if (geh::check_plan_args(m, n, k, dt, ep, GE_OP_N, GE_OP_N, &lay) != GE_OK) return;
  const int chosen = geh::choose_cfg(m, n, k, t, cus, lay);
  for (int cfg = 0; cfg < gek::CFG_COUNT; ++cfg) {
    for (int split = 0; split < 2; ++split) {
      geh::Layout L;
      const ge_status_t st = geh::make_layout(m, n, k, dt, ep, lay, cus, cfg, split != 0, true, &L);
      if (t == GE_F32 && gek::cfg_is_dtl(cfg)) {
        check(st == GE_ERR_NOT_SUPPORTED, "fp32 has no direct-to-LDS tiles", m, n, k, cfg);
        continue;
      }
      check(st == GE_OK, "layout", m, n, k, cfg);
      if (st != GE_OK) continue;
      const gek::TileCfg& tc = gek::kTiles[cfg];
      check((long long)L.tiles_m * tc.bm >= m && (long long)(L.tiles_m - 1) * tc.bm < m, "m tiles", m, n, k, cfg);
      check((long long)L.tiles_n * tc.bn >= n && (long long)(L.tiles_n - 1) * tc.bn < n, "n tiles", m, n, k, cfg);
      const int tiles = L.tiles_m * L.tiles_n;
      check(L.dp_tiles <= tiles && (L.sk_wgs == 0) == (L.dp_tiles == tiles), "split bookkeeping", m, n, k, cfg);
      if (!split) check(L.sk_wgs == 0, "no split when not allowed", m, n, k, cfg);
      if (L.persist_grid) {
        check(gek::cfg_can_persist(cfg) && L.sk_wgs == 0 && L.persist_grid == (tiles < cus ? tiles : cus), "persistent grid", m,
              n, k, cfg);
        check(k % tc.bk == 0 && (k / tc.bk) % tc.stages == 0 && k / tc.bk >= 2 * tc.stages, "persistent k loop", m,
              n, k, cfg);
      }
      // workspace regions
      std::vector<std::pair<size_t, size_t>> regions;
      if (L.sk_wgs) regions.push_back({L.off_sk_flag, L.sk_flag_bytes});
      if (ep == GE_EPILOG_DRELU_BGRAD) regions.push_back({L.off_partial, (size_t)L.partial_cols * (size_t)m * 4});
      if (ep == GE_EPILOG_RELU_BIAS_UNFUSED) {
        const size_t es = geh::elem_size(t);
        regions.push_back({L.off_t1, (size_t)m * (size_t)n * es});
        regions.push_back({L.off_t2, (size_t)m * (size_t)n * es});
      }
      if (ep == GE_EPILOG_DRELU_BGRAD_UNFUSED) regions.push_back({L.off_t1, (size_t)m * (size_t)n * geh::elem_size(t)});
      if (L.sk_wgs) regions.push_back({L.off_sk_partial, (size_t)L.sk_wgs * gek::sk_slot_bytes(tc)});
      for (size_t i = 0; i < regions.size(); ++i) {
        check(regions[i].first % 16 == 0, "region aligned", m, n, k, cfg);
        check(regions[i].first + regions[i].second <= L.ws_bytes, "region inside the workspace", m, n, k, cfg);
        for (size_t j = i + 1; j < regions.size(); ++j)
          check(regions[i].first + regions[i].second <= regions[j].first ||
                    regions[j].first + regions[j].second <= regions[i].first,
                "regions disjoint", m, n, k, cfg);
      }
      if (L.sk_wgs) {
        check(L.off_sk_flag == 0 && L.sk_flag_bytes == geh::kSkFlagRegion && L.sk_wgs < gek::kSkLostWord,
              "flag region first; flags clear of the lost-wait count", m, n, k, cfg);
        check_split(L, (int)((k + tc.bk - 1) / tc.bk), cus, m, n, k);
      }
      const std::string d = geh::describe(dt, ep, L);
      check(!d.empty(), "description", m, n, k, cfg);
    }
  }
  check(chosen >= 0 && chosen < gek::CFG_COUNT, "chosen configuration", m, n, k, chosen);
}

}  // namespace

int main() {
  check_args();
  const long long ms[] = {1, 33, 200, 1024, 1032, 4096, 4352, 8192, 12000, 65536};
  const long long ns[] = {8, 136, 512, 1376, 4096, 11008};
  const long long ks[] = {8, 72, 256, 2048, 4096, 8192};
  const ge_epilog_t eps[] = {GE_EPILOG_RELU_BIAS, GE_EPILOG_DRELU_BGRAD, GE_EPILOG_RELU_BIAS_UNFUSED,
                             GE_EPILOG_DRELU_BGRAD_UNFUSED};
  const int cuss[] = {256, 80, 1};
  int cases = 0;
  for (long long m : ms)
    for (long long n : ns)
      for (long long k : ks)
        for (ge_epilog_t ep : eps)
          for (int cus : cuss)
            for (ge_dtype_t t : {GE_F16, GE_F32}) {
              if (geh::is_unfused(ep) && m * n > (1LL << 26)) continue;   // keep the run short
              check_layout(m, n, k, t, ep, cus);
              ++cases;
            }
  std::printf("%d problems; ok (%d failures)\n", cases, failures);
  return failures ? 1 : 0;
}
