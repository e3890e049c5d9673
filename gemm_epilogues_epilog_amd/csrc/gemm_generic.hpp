// Generic fused kernel: register-staged global -> LDS copies. Used for fp32 and for
// tiles too small for the direct-to-LDS kernel; any storage type, any tile shape
// that satisfies the static checks below.
#pragma once

#include "kernels.hpp"

namespace gek {

// ---- the fused kernel ----------------------------------------------------------

template <int DT, int EP, int BM, int BN, int WM, int WN>
struct Cfg {
  using T = Tr<DT>;
  static constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN;
  static constexpr int NW = WAVES_M * WAVES_N, NT = NW * 64;
  static constexpr int MB = WM / 32, NB = WN / 32;
  static constexpr int E = T::E, es = T::es;
  static constexpr int BK = kRowBytes / es;              // k per tile (= 8 E)
  static constexpr int STAGE = (BM + BN) * kRowBytes;    // LDS bytes per stage
  static constexpr int A_LD = BM * 8 / NT;               // A chunks per thread per tile
  // B: each thread transposes R k-rows x E columns; B_LD such blocks per tile
  static constexpr int R0 = 8 * BN / NT;
  static constexpr int R = R0 < E ? R0 : E;
  static constexpr int B_LD = 8 * BN / (NT * R);
  static constexpr int NBN = BN / E;                     // E-wide column blocks of the B tile
  static constexpr int KSTEPS = kRowBytes / 32;          // k-steps (two chunks each) per tile
  static_assert(BM % WM == 0 && BN % WN == 0 && WM % 32 == 0 && WN % 32 == 0, "tile shape");
  static_assert((BM * 8) % NT == 0 && A_LD >= 1, "A tile split");
  static_assert(R >= 1 && (DT == F32 || R >= 2) && E % R == 0 && B_LD >= 1 && (8 * BN) % (NT * R) == 0,
                "B tile split");
};

template <int DT, int EP, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64, 1) void gemm_epilog_kernel(Args p) {
  using C = Cfg<DT, EP, BM, BN, WM, WN>;
  using T = typename C::T;
  constexpr int NT = C::NT, E = C::E, es = C::es, R = C::R;
  constexpr int MB = C::MB, NB = C::NB;

  __shared__ __attribute__((aligned(16))) char lds[2 * C::STAGE];

  const int64_t M = p.m;
  const int N = p.n, K = p.k;

  int tm, tn;
  tile_coords(p, tm, tn);
  const int64_t m0 = (int64_t)tm * BM;
  const int n0 = tn * BN;

  const int t = threadIdx.x;
  const int lane = t & 63, w = t >> 6;
  const int wm = w % C::WAVES_M, wn = w / C::WAVES_M;
  const int lrow = lane & 31, lhi = lane >> 5;

  // ---- global -> register load plan -----------------------------------------
  const int a_ch = t & 7;                      // chunk of the A row this thread copies
  uint32_t a_off[C::A_LD];
  int a_lds[C::A_LD];
#pragma unroll
  for (int i = 0; i < C::A_LD; ++i) {
    const int row = (t + i * NT) >> 3;
    a_off[i] = (m0 + row < M) ? (uint32_t)(row * K * es + a_ch * 16) : kOOB;
    a_lds[i] = row * kRowBytes + ((a_ch ^ (row & 7)) << 4);
  }
  uint32_t b_off[C::B_LD];
  int b_kr[C::B_LD];       // first k-row of the block inside the tile
  int b_nc[C::B_LD];       // first column of the block inside the tile
#pragma unroll
  for (int i = 0; i < C::B_LD; ++i) {
    const int q = t + i * NT;
    const int nb = q % C::NBN, kb = q / C::NBN;
    b_kr[i] = kb * R;
    b_nc[i] = nb * E;
    b_off[i] = (n0 + nb * E < N) ? (uint32_t)(kb * R * N * es + nb * 16) : kOOB;
  }

  const char* Abase = static_cast<const char*>(p.A) + m0 * (int64_t)K * es;
  const char* Bbase = static_cast<const char*>(p.B) + (int64_t)n0 * es;
  const int KT = (K + C::BK - 1) / C::BK;

  i32x4 areg[C::A_LD];
  i32x4 breg[C::B_LD][R];

  auto load_tile = [&](int kt) {
    const int k0 = kt * C::BK;
    const __amdgpu_buffer_rsrc_t ra = rsrc(Abase + (int64_t)kt * kRowBytes);
    const __amdgpu_buffer_rsrc_t rb = rsrc(Bbase + (int64_t)k0 * N * es);
    const bool a_kok = k0 + a_ch * E < K;
#pragma unroll
    for (int i = 0; i < C::A_LD; ++i)
      areg[i] = __builtin_amdgcn_raw_buffer_load_b128(ra, a_kok ? a_off[i] : kOOB, 0, 0);
#pragma unroll
    for (int i = 0; i < C::B_LD; ++i) {
#pragma unroll
      for (int kk = 0; kk < R; ++kk) {
        const bool kok = k0 + b_kr[i] + kk < K;
        breg[i][kk] = __builtin_amdgcn_raw_buffer_load_b128(rb, kok ? b_off[i] + (uint32_t)(kk * N * es) : kOOB, 0, 0);
      }
    }
  };

  auto store_tile = [&](int stage) {
    char* sA = lds + stage * C::STAGE;
    char* sB = sA + BM * kRowBytes;
#pragma unroll
    for (int i = 0; i < C::A_LD; ++i) *reinterpret_cast<i32x4*>(sA + a_lds[i]) = areg[i];
#pragma unroll
    for (int i = 0; i < C::B_LD; ++i) {
      // transpose R rows x E columns into E columns x R k-values
      const int kbyte = b_kr[i] * es;                 // byte offset of the k-run in an LDS row
      const int chunk = kbyte >> 4, within = kbyte & 15;
#pragma unroll
      for (int c = 0; c < E; ++c) {
        const int row = b_nc[i] + c;
        char* dst = sB + row * kRowBytes + ((chunk ^ (row & 7)) << 4) + within;
        if constexpr (es == 4) {
          if constexpr (R == 4) {
            i32x4 v = {breg[i][0][c], breg[i][1][c], breg[i][2][c], breg[i][3][c]};
            *reinterpret_cast<i32x4*>(dst) = v;
          } else if constexpr (R == 2) {
            i32x2 v = {breg[i][0][c], breg[i][1][c]};
            *reinterpret_cast<i32x2*>(dst) = v;
          } else {
            *reinterpret_cast<int*>(dst) = breg[i][0][c];
          }
        } else {
          // 16-bit: column c sits in dword c/2 of every row, low half for even c
          const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
          uint32_t d[R / 2];
#pragma unroll
          for (int e = 0; e < R / 2; ++e)
            d[e] = __builtin_amdgcn_perm((uint32_t)breg[i][2 * e + 1][c >> 1], (uint32_t)breg[i][2 * e][c >> 1], sel);
          if constexpr (R == 8) {
            i32x4 v = {(int)d[0], (int)d[1], (int)d[2], (int)d[3]};
            *reinterpret_cast<i32x4*>(dst) = v;
          } else if constexpr (R == 4) {
            i32x2 v = {(int)d[0], (int)d[1]};
            *reinterpret_cast<i32x2*>(dst) = v;
          } else {
            *reinterpret_cast<int*>(dst) = (int)d[0];
          }
        }
      }
    }
  };

  f32x16 acc[NB][MB];
#pragma unroll
  for (int a = 0; a < NB; ++a)
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

  // ---- main loop: double-buffered LDS, one barrier per k-tile ----------------
  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) load_tile(kt + 1);
    const char* sA = lds + cur * C::STAGE + (wm * WM + lrow) * kRowBytes;
    const char* sB = lds + cur * C::STAGE + BM * kRowBytes + (wn * WN + lrow) * kRowBytes;
#pragma unroll
    for (int s = 0; s < C::KSTEPS; ++s) {
      const int phys = ((2 * s + lhi) ^ (lrow & 7)) << 4;
      i32x4 af[MB], bf[NB];
#pragma unroll
      for (int b = 0; b < MB; ++b) af[b] = *reinterpret_cast<const i32x4*>(sA + b * 32 * kRowBytes + phys);
#pragma unroll
      for (int a = 0; a < NB; ++a) bf[a] = *reinterpret_cast<const i32x4*>(sB + a * 32 * kRowBytes + phys);
#pragma unroll
      for (int a = 0; a < NB; ++a)
#pragma unroll
        for (int b = 0; b < MB; ++b) acc[a][b] = T::mma(bf[a], af[b], acc[a][b]);
    }
    if (kt + 1 < KT) store_tile(cur ^ 1);
    __syncthreads();
  }

  epilogue<DT, EP, MB, NB, WN>(p, acc, m0 + wm * WM, n0 + wn * WN, lane);
}


}  // namespace gek
