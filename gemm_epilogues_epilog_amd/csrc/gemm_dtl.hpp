// Fused kernel for fp16 / bf16 with direct-to-LDS operand copies (gfx950).
//
// Per k-tile (64 values of k) every wave issues buffer loads that write straight
// into LDS (no register staging, no VALU work on the copy path):
//   A tile: BM rows of 128 bytes (row = m, k contiguous), the eight 16-byte chunks
//           of each row XOR-swizzled by swz_a(row).
//   B tile: 64 rows of 2 BN bytes (row = k, n contiguous, as B is stored), the
//           16-byte chunks XOR-swizzled by swz_b(row).
// Fragments: A with ds_read_b128 (8 consecutive k of one row), B with two
// ds_read_b64_tr_b16 per fragment. In each 16-lane group of that instruction lane j
// receives, as element q, the (j % 4)-th 16-bit value of the 8 bytes read by group
// lane 4q + j/4; when group lane i reads row k0 + i/4 at columns 4 (i % 4) .. +3,
// lane j therefore holds column j at rows k0 .. k0+3, which is the MFMA operand
// layout (k contiguous per lane) produced from the n-contiguous tile.
//
// Both LDS stages are filled one k-tile ahead; one barrier per k-tile separates
// "everyone finished reading stage s" from "stage s is refilled". Fragment
// registers are double-buffered so the reads of k-step s+1 overlap the MFMAs of
// k-step s.
#pragma once

#include "kernels.hpp"

namespace gek {

// 16-byte chunk swizzles. A rows are 128 bytes (8 chunks): rows r .. r+15 read at
// the same logical chunk hit 16 distinct 16-byte bank groups whether the LDS
// serves 8 or 16 lanes of a ds_read_b128 per cycle. Depends on row % 16 only.
__device__ __forceinline__ int swz_a(int row) { return (row & 7) ^ ((row >> 3) & 1); }
// B rows are 2 BN bytes. A transposed read touches rows k0 .. k0+3 (k0 % 4 == 0) at
// the same 32 columns; XOR with g in {0, 6, 10, 12} puts those rows in distinct
// 32-byte and 64-byte bank groups.
__device__ __forceinline__ int swz_b(int row) {
  const int u = row & 3;
  return u == 0 ? 0 : u == 1 ? 6 : u == 2 ? 10 : 12;
}

typedef short s16x4 __attribute__((__vector_size__(4 * sizeof(short))));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ i32x2 ds_read_tr(const char* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(i32x2, v);
}

template <int DT, int EP, int BM, int BN, int WM, int WN>
struct DtlCfg {
  static constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN;
  static constexpr int NW = WAVES_M * WAVES_N, NT = NW * 64;
  static constexpr int MB = WM / 32, NB = WN / 32;
  static constexpr int BK = 64;                          // k per tile (128 bytes of fp16/bf16)
  static constexpr int A_BYTES = BM * kRowBytes;
  static constexpr int B_ROWB = BN * 2;                  // bytes per B row in LDS
  static constexpr int B_BYTES = BK * B_ROWB;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int A_INST = A_BYTES / 1024 / NW;     // 1 KB direct-to-LDS copies per wave
  static constexpr int B_INST = B_BYTES / 1024 / NW;
  static constexpr int B_CHUNKS = B_ROWB / 16;           // 16-byte chunks per B row
  static constexpr int B_RPI = 1024 / B_ROWB;            // B rows per copy instruction
  static_assert(DT == F16 || DT == BF16, "16-bit types only");
  static_assert(BN >= 128 && BN % 64 == 0, "B rows must hold at least 16 chunks");
  static_assert(A_BYTES % (1024 * NW) == 0 && B_BYTES % (1024 * NW) == 0, "copy split");
  static_assert(2 * STAGE <= 160 * 1024, "LDS");
};

template <int DT, int EP, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64, 1) void gemm_dtl_kernel(Args p) {
  using C = DtlCfg<DT, EP, BM, BN, WM, WN>;
  using T = Tr<DT>;
  constexpr int MB = C::MB, NB = C::NB;

  // One LDS object per stage: the compiler then knows that copies in flight into
  // one stage do not alias fragment reads of the other and waits only where needed.
  __shared__ __attribute__((aligned(1024))) char stage0[C::STAGE];
  __shared__ __attribute__((aligned(1024))) char stage1[C::STAGE];

  const int64_t M = p.m;
  const int N = p.n, K = p.k;
  int tm, tn;
  tile_coords(p, tm, tn);
  const int64_t m0 = (int64_t)tm * BM;
  const int n0 = tn * BN;

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = w % C::WAVES_M, wn = w / C::WAVES_M;
  const int lrow = lane & 31, lhi = lane >> 5;

  // ---- copy plan: per-lane source offsets (tile-relative, constant over k) ----
  uint32_t a_src[C::A_INST];
  int a_chunk[C::A_INST];
#pragma unroll
  for (int j = 0; j < C::A_INST; ++j) {
    const int row = (w * C::A_INST + j) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ swz_a(row);
    a_chunk[j] = c;
    a_src[j] = (m0 + row < M) ? (uint32_t)(row * K * 2 + c * 16) : kOOB;
  }
  uint32_t b_src[C::B_INST];
  int b_row[C::B_INST];
#pragma unroll
  for (int j = 0; j < C::B_INST; ++j) {
    const int row = (w * C::B_INST + j) * C::B_RPI + lane / C::B_CHUNKS;
    const int c = (lane % C::B_CHUNKS) ^ swz_b(row);
    b_row[j] = row;
    b_src[j] = (n0 + c * 8 < N) ? (uint32_t)(row * N * 2 + c * 16) : kOOB;
  }

  const char* Abase = static_cast<const char*>(p.A) + m0 * (int64_t)K * 2;
  const char* Bbase = static_cast<const char*>(p.B) + (int64_t)n0 * 2;
  const int KT = (K + C::BK - 1) / C::BK;

  auto issue_copies = [&](int kt, char* st) {
    const int k0 = kt * C::BK;
    const __amdgpu_buffer_rsrc_t ra = rsrc(Abase + (int64_t)k0 * 2);
    const __amdgpu_buffer_rsrc_t rb = rsrc(Bbase + (int64_t)k0 * N * 2);
    char* sA = st;
    char* sB = sA + C::A_BYTES;
    const bool tail = k0 + C::BK > K;
#pragma unroll
    for (int j = 0; j < C::A_INST; ++j) {
      const uint32_t off = (tail && k0 + a_chunk[j] * 8 >= K) ? kOOB : a_src[j];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(sA + (w * C::A_INST + j) * 1024), 16, off, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < C::B_INST; ++j) {
      const uint32_t off = (tail && k0 + b_row[j] >= K) ? kOOB : b_src[j];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(sB + (w * C::B_INST + j) * 1024), 16, off, 0, 0, 0);
    }
  };

  // ---- fragment read addresses (stage-relative) -----------------------------
  int a_rd[4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
    a_rd[s] = (wm * WM + lrow) * kRowBytes + (((2 * s + lhi) ^ swz_a(lrow)) << 4);
  int b_rd[NB];
  {
    const int g = lane >> 4, i = lane & 15;
    const int row = 8 * lhi + (i >> 2);              // + 16 s + 4 t
#pragma unroll
    for (int a = 0; a < NB; ++a) {
      const int n = wn * WN + a * 32 + 16 * (g & 1) + 4 * (i & 3);
      b_rd[a] = C::A_BYTES + row * C::B_ROWB + (((n >> 3) ^ swz_b(row)) << 4) + ((n & 7) << 1);
    }
  }

  f32x16 acc[NB][MB];
#pragma unroll
  for (int a = 0; a < NB; ++a)
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

  i32x4 fa[2][MB];
  i32x4 fb[2][NB];
  auto read_frags = [&](const char* base, int s, int buf) {
#pragma unroll
    for (int b = 0; b < MB; ++b) fa[buf][b] = *reinterpret_cast<const i32x4*>(base + a_rd[s] + b * 32 * kRowBytes);
#pragma unroll
    for (int a = 0; a < NB; ++a) {
      const char* q = base + b_rd[a] + 16 * s * C::B_ROWB;
      const i32x2 lo = ds_read_tr(q);
      const i32x2 hi = ds_read_tr(q + 4 * C::B_ROWB);
      fb[buf][a] = i32x4{lo[0], lo[1], hi[0], hi[1]};
    }
  };

  // ---- prologue: tiles 0 and 1 in flight, tile 0 complete -------------------
  issue_copies(0, stage0);
  if (KT > 1) issue_copies(1, stage1);
  if (KT > 1) {
    wait_vmcnt<C::A_INST + C::B_INST>();   // tile 0 landed, tile 1 may be in flight
  } else {
    wait_vmcnt<0>();
  }
  __syncthreads();
  read_frags(stage0, 0, 0);

  // One k-tile on stage `cur` (the other stage holds or receives tile kt+1).
  auto tile = [&](int kt, char* cur, char* nxt) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int buf = s & 1;
      if (s < 3) {
        read_frags(cur, s + 1, buf ^ 1);
      } else {
        // step 3 is in registers: once every wave is here, `cur` may be refilled;
        // the barrier's wait also makes tile kt+1 (in `nxt`) complete
        __syncthreads();
        if (kt + 2 < KT) issue_copies(kt + 2, cur);
        if (kt + 1 < KT) read_frags(nxt, 0, 0);
      }
#pragma unroll
      for (int a = 0; a < NB; ++a)
#pragma unroll
        for (int b = 0; b < MB; ++b) acc[a][b] = T::mma(fb[buf][a], fa[buf][b], acc[a][b]);
      // keep each k-step's reads next to its MFMAs (no hoisting across steps)
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  for (int kt = 0; kt < KT; kt += 2) {
    tile(kt, stage0, stage1);
    if (kt + 1 < KT) tile(kt + 1, stage1, stage0);
  }

  epilogue<DT, EP, MB, NB, WN>(p, acc, m0 + wm * WM, n0 + wn * WN, lane);
}

}  // namespace gek
