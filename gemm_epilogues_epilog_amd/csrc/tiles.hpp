// Kernel-configuration table and split-tail run arithmetic, shared by the host plan
// (plan_host.cpp, plain C++) and the kernels. Everything here is constexpr: the host
// compiler evaluates it for the plan, and in HIP device code constexpr functions are
// callable as they are, so the kernels and the plan use one definition.
#pragma once

#include <cstddef>
#include <cstdint>

namespace gek {

// Workgroup tile (BM x BN), wave tile (WM x WN), k-tile and LDS stages of each
// configuration. S and M use the register-staged kernel (any type); the L family
// uses the direct-to-LDS kernel (16-bit types only).
struct TileCfg {
  int bm, bn, wm, wn, bk, stages;
  const char* name;
  const char* loop;   // main loop of the direct-to-LDS kernels
};

enum CfgId { CFG_S = 0, CFG_M, CFG_L, CFG_LH, CFG_LM, CFG_LM4, CFG_LMD, CFG_L3, CFG_LW, CFG_COUNT };

constexpr TileCfg kTiles[CFG_COUNT] = {
    {64, 64, 32, 32, 0, 2, "S", ""},
    {128, 128, 64, 64, 0, 2, "M", ""},
    {256, 256, 128, 64, 64, 2, "L", "persistent lockstep interleaved, copies on waves 0-3"},   // 8 waves (default)
    {256, 256, 128, 64, 64, 2, "LH", "lockstep, copies on waves 0-3"},
    {128, 128, 32, 64, 64, 2, "LM", "lockstep"},                        // 8 waves of 32 x 64, two per CU
    {128, 128, 64, 64, 64, 2, "LM4", "lockstep"},                       // 4 waves of 64 x 64, two per CU
    {128, 128, 32, 64, 64, 3, "LMD", "lockstep"},                       // LM with a 3-stage ring, one per CU
    {192, 256, 96, 64, 64, 2, "L3", "persistent lockstep interleaved, copies on waves 0-3"},   // 8 waves of 96 x 64
    {128, 256, 64, 64, 64, 2, "LW", "persistent lockstep interleaved, copies on waves 0-3"},   // 8 waves of 64 x 64
};

constexpr bool cfg_is_dtl(int c) { return c >= CFG_L; }
// Configurations whose kernel can split the last round's K loop (8-wave lockstep
// loops; the 4-wave tile has no registers left for the partial sums).
constexpr bool cfg_can_split(int c) {
  return (c >= CFG_L && c <= CFG_LM) || c == CFG_LMD || c == CFG_L3 || c == CFG_LW;
}
// Configurations with a persistent kernel, used when the tile grid is not split and
// k spans a whole number of stage rings, at least two.
constexpr bool cfg_can_persist(int c) { return c == CFG_L || c == CFG_L3 || c == CFG_LW; }
// Configurations with kernels for operands stored transposed (16-bit types): the
// 256 x 256 tile persistent (L) or with copies on waves 0-3 (LH), and the 128 x 128
// tile (LM).
constexpr bool cfg_has_layouts(int c) { return c == CFG_L || c == CFG_LH || c == CFG_LM || c == CFG_LMD; }

// The split tail's flag words at the start of a workspace: one per split workgroup
// (fewer than kSkFlagWords - 1) and, in the last word, the count of owner waits that
// ran out. Both sit at fixed places, so a workspace reused by problems of different
// layouts never finds a count where a flag belongs.
constexpr int kSkFlagWords = 1024;
constexpr int kSkLostWord = kSkFlagWords - 1;

// Partial-accumulator bytes of one split workgroup of a configuration (one tile, fp32).
constexpr size_t sk_slot_bytes(const TileCfg& c) { return (size_t)c.bm * c.bn * sizeof(float); }

// ---- split tail: the pieces of one run ---------------------------------------------
// The tail tiles' k-tiles are numbered u = t * KT + kk over (tail tile t, k-tile kk)
// and cut into runs of `units` (< KT) consecutive numbers, one workgroup per run.
// Run r covers [r units, min(total, (r+1) units)). Because units < KT a run holds at
// most one tile start, so it splits into at most two pieces:
//   the partial piece before that start (a tile's k-tiles from kb > 0 on), whose fp32
//   sums the run publishes;
//   the owner piece from the start on (k-tiles 0 .. own_nt - 1 of tile own_t), whose
//   workgroup adds the partials of runs r+1 .. last and runs the epilogue.
struct SkRun {
  int pa_t, pa_kb, pa_nt;   // partial piece: tail tile, first k-tile, k-tiles (0: none)
  int own_t, own_nt;        // owner piece: tail tile, k-tiles from 0 (0: none)
  int last;                 // owner: last run holding a part of tile own_t
};

constexpr SkRun sk_run(int r, int units, int kt, int tail_tiles, int wgs) {
  SkRun s{0, 0, 0, 0, 0, 0};
  const int total = tail_tiles * kt;
  const int u0 = r * units;
  const int u1 = total < u0 + units ? total : u0 + units;
  const int ts = (u0 + kt - 1) / kt * kt;   // first tile start at or after u0
  const int pend = ts < u1 ? ts : u1;
  if (u0 < pend) {
    s.pa_t = u0 / kt;
    s.pa_kb = u0 - s.pa_t * kt;
    s.pa_nt = pend - u0;
  }
  s.own_t = ts / kt;
  s.own_nt = u1 - ts > 0 ? u1 - ts : 0;
  const int lr = ((s.own_t + 1) * kt - 1) / units;
  s.last = lr < wgs - 1 ? lr : wgs - 1;
  return s;
}

}  // namespace gek
