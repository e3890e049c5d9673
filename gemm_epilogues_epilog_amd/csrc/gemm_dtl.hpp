// Fused kernel for fp16 / bf16 with direct-to-LDS operand copies (gfx950).
//
// Operands. Per k-tile (BK values of k) the copying waves (all, or one per SIMD)
// issue buffer loads that write straight into LDS (no register staging, no VALU work
// on the copy path):
//   A tile: BM rows of 2 BK bytes (row = m, k contiguous), the 16-byte chunks of
//           each row XOR-swizzled by swz_a(row).
//   B tile: BK rows of 2 BN bytes (row = k, n contiguous, as B is stored), the
//           16-byte chunks XOR-swizzled by swz_b(row).
// Fragments: A with ds_read_b128 (8 consecutive k of one row), B with two
// ds_read_b64_tr_b16 per fragment. In each 16-lane group of that instruction lane j
// receives, as element q, the (j % 4)-th 16-bit value of the 8 bytes read by group
// lane 4q + j/4; when group lane i reads row k0 + i/4 at columns 4 (i % 4) .. +3,
// lane j therefore holds column j at rows k0 .. k0+3, which is the MFMA operand
// layout (k contiguous per lane) produced from the n-contiguous tile.
//
// Pipeline. STAGES LDS stages form a ring. The copies are inline assembly, ordered
// by hand with vmcnt / lgkmcnt waits and workgroup barriers (the lockstep and
// persistent loops below describe their schedules): the compiler would otherwise
// make every LDS read wait for every copy still in flight.
//
// Epilogue. Each wave writes its finished (activated, rounded) accumulators to LDS
// scratch with a swizzle that keeps the 8-byte writes conflict-free, reads them back
// as 16-byte row pieces and stores whole 2 WN-byte row segments of D, so every store
// instruction covers full cache lines instead of 32 rows x 16 bytes. One-tile kernels
// use the freed stage memory for the whole WM x WN tile (epilogue_lds); the
// persistent kernel keeps 32 rows per wave of its own, block by block
// (epilogue_block), since the stages then hold the next tile's operands.
#pragma once

#include <type_traits>

#include "kernels.hpp"
#include "tiles.hpp"

namespace gek {

typedef short s16x4 __attribute__((__vector_size__(4 * sizeof(short))));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ i32x2 ds_read_tr(const char* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(i32x2, v);
}

// 16-byte chunk swizzle of A rows. A ds_read_b128 is served 16 lanes (256 bytes) at
// a time; lanes 0-15 read rows r .. r+15 (r % 16 == 0) at one logical chunk, which
// must land in 16 distinct 16-byte bank groups.
//   128-byte rows (8 chunks): bank group = 8 (row % 2) + chunk; XOR with a value
//     that differs across the 8 rows of equal parity.
//   64-byte rows (4 chunks): bank group = 4 (row % 4) + chunk; XOR with row / 4.
template <int ROWB>
__device__ __forceinline__ int swz_a(int row) {
  static_assert(ROWB == 64 || ROWB == 128, "A row bytes");
  if constexpr (ROWB == 128) return (row & 7) ^ ((row >> 3) & 1);
  else return (row >> 2) & 3;
}
// B rows are 2 BN bytes. A transposed read touches rows k0 .. k0+3 (k0 % 4 == 0) at
// the same 32 columns; XOR with g in {0, 6, 10, 12} puts those rows in distinct
// 32-byte and 64-byte bank groups.
__device__ __forceinline__ int swz_b(int row) {
  const int u = row & 3;
  return u == 0 ? 0 : u == 1 ? 6 : u == 2 ? 10 : 12;
}

// CW: how many waves (the first CW) issue the operand copies; 0 = all of them.
template <int BM, int BN, int WM, int WN, int BK, int STAGES, int CW_ = 0>
struct DtlCfg {
  static constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN;
  static constexpr int NW = WAVES_M * WAVES_N, NT = NW * 64;
  static constexpr int CW = CW_ ? CW_ : NW;
  static constexpr int MB = WM / 32, NB = WN / 32;
  static constexpr int KSTEPS = BK / 16;                  // MFMA k-steps per tile
  static constexpr int A_ROWB = BK * 2;                   // bytes per A row in LDS
  static constexpr int A_BYTES = BM * A_ROWB;
  static constexpr int A_CHUNKS = A_ROWB / 16;
  static constexpr int A_RPI = 1024 / A_ROWB;             // A rows per copy instruction
  static constexpr int B_ROWB = BN * 2;                   // bytes per B row in LDS
  static constexpr int B_BYTES = BK * B_ROWB;
  static constexpr int B_CHUNKS = B_ROWB / 16;
  static constexpr int B_RPI = 1024 / B_ROWB;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int A_INST = A_BYTES / 1024 / CW;      // 1 KB copies per copy wave per tile
  static constexpr int B_INST = B_BYTES / 1024 / CW;
  static constexpr int INST = A_INST + B_INST;
  static constexpr int SCRATCH = WM * WN * 2;             // epilogue bytes per wave
  static constexpr int LDS = STAGES * STAGE;
  static_assert(BK == 32 || BK == 64, "k-tile");
  static_assert(BN >= 128 && BN % 64 == 0, "B rows must hold at least 16 chunks");
  static_assert(CW >= 1 && CW <= NW, "copy waves");
  static_assert(A_BYTES % (1024 * CW) == 0 && B_BYTES % (1024 * CW) == 0, "copy split");
  static_assert(STAGES >= 2 && LDS <= 160 * 1024, "LDS");
  static_assert(NW * SCRATCH <= LDS, "epilogue scratch");
  static_assert((STAGES - 2) * INST < 64, "vmcnt range");
};

// s_waitcnt vmcnt(n * INST) for a run-time n in [0, MAXN] (larger n waits for MAXN).
template <int INST, int MAXN>
__device__ __forceinline__ void wait_tiles(int n) {
  if constexpr (MAXN <= 0) {
    wait_vmcnt<0>();
  } else {
    if (n >= MAXN) wait_vmcnt<MAXN * INST>();
    else wait_tiles<INST, MAXN - 1>(n);
  }
}

// ---- epilogue through LDS ------------------------------------------------------
// D is stored with the non-temporal cache policy (bit nt of a buffer instruction), as a
// stream that nothing in the kernel reads back. Measured A/B in one call: 7B-FFN
// headline 0.7% faster, 8192^3 bf16 forward 1.5%, the 8192 training step 0.8%, the
// unfused chain (which reads its intermediate back) 0.6%. The operand bytes fetched past
// the L2 do not change (FETCH_SIZE), so the gain is in how the stores drain.
constexpr int kStreamStore = 2;
// The accumulators (lane l: row 32 b + l % 32 of the wave tile, columns
// 32 a + 8 (r / 4) + 4 (l / 32) + r % 4) are finished in registers and written to
// the wave's scratch as 8-byte units: unit p of row `row` goes to unit
// p ^ swz(row), where swz spreads the 32 rows written by one half-wave over all 32
// 8-byte bank slots. Read-back takes 16 bytes (units 2c, 2c+1 -> stored at the
// aligned pair 2 (c ^ (s >> 1)), in swapped order when s is odd).
template <int WN>
struct EpiLayout {
  static constexpr int RB = WN * 2;          // scratch row bytes
  static constexpr int U = RB / 8;           // 8-byte units per row
  static constexpr int LPR = RB / 16;        // lanes per row on read-back
  static constexpr int RPI = 64 / LPR;       // rows per read-back instruction
  static_assert(U == 16 || U == 32, "scratch row");
  __device__ static __forceinline__ int swz(int row) { return U == 16 ? ((row >> 1) & 15) : (row & 31); }
};

template <int DT, int EP, int MB, int NB, int WN>
__device__ __forceinline__ void epilogue_lds(const Args& p, f32x16 (&acc)[NB][MB], int64_t m0w, int n0w, int lane,
                                             char* scratch) {
  using T = Tr<DT>;
  using L = EpiLayout<WN>;
  constexpr int WM = MB * 32;
  const int64_t M = p.m;
  const int N = p.n;
  const int lrow = lane & 31, lhi = lane >> 5;

  // ---- phase 1: finish every accumulator and stage it in scratch ----
  if constexpr (EP == DRELU_BGRAD) {
#pragma unroll
    for (int b = 0; b < MB; ++b) {
      const int row = 32 * b + lrow;
      const int64_t mrow = m0w + row;
      const int64_t grp = (m0w + 32 * b) >> 5;
      const bool gok = grp * 32 < M;
      const int s = L::swz(row);
      float rowsum = 0.0f;
#pragma unroll
      for (int a = 0; a < NB; ++a) {
        const int ncol = n0w + 32 * a + lrow;
        uint32_t word = 0;
        if (gok && ncol < N) word = p.aux[grp * N + ncol];
        float dz[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          dz[r] = mask_bit_of_reg(word, r) ? acc[a][b][r] : 0.0f;
          rowsum += dz[r];
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int unit = (8 * a + 2 * g + lhi) ^ s;
          const i32x2 v = {(int)T::pack2(dz[4 * g], dz[4 * g + 1]), (int)T::pack2(dz[4 * g + 2], dz[4 * g + 3])};
          *reinterpret_cast<i32x2*>(scratch + row * L::RB + unit * 8) = v;
        }
      }
      rowsum += __shfl_xor(rowsum, 32);
      if (lhi == 0 && mrow < M && n0w < N) p.partial[(int64_t)(n0w / WN) * M + mrow] = rowsum;
    }
  } else {
#pragma unroll
    for (int b = 0; b < MB; ++b) {
      const int row = 32 * b + lrow;
      const int64_t mrow = m0w + row;
      const bool mok = mrow < M;
      const int s = L::swz(row);
      float bv = 0.0f;
      if constexpr (EP != NONE) {
        if (mok) bv = load_vec(p.bias, p.vec_dt, mrow);
      }
#pragma unroll
      for (int a = 0; a < NB; ++a) {
        float pre[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) pre[r] = acc[a][b][r] + bv;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float y[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = activate<EP>(pre[4 * g + e]);
          const int unit = (8 * a + 2 * g + lhi) ^ s;
          const i32x2 v = {(int)T::pack2(y[0], y[1]), (int)T::pack2(y[2], y[3])};
          *reinterpret_cast<i32x2*>(scratch + row * L::RB + unit * 8) = v;
        }
        if constexpr (EP == RELU_AUX_BIAS) {
          const uint32_t word = relu_mask_words(pre, mok);
          const int64_t grp = (m0w + 32 * b) >> 5;
          const int ncol = n0w + 32 * a + lane;
          if (lane < 32 && grp * 32 < M && ncol < N) p.aux[grp * N + ncol] = word;
        }
      }
    }
  }

  // ---- phase 2: whole row segments from scratch to D ----
  char* Dw = static_cast<char*>(p.D) + (m0w * (int64_t)N + n0w) * 2;
  const __amdgpu_buffer_rsrc_t rd = rsrc(Dw);
  const int c = lane % L::LPR;
  const bool cok = n0w + 8 * c < N;
  // read-backs in groups of four ahead of their stores: the compiler does not move an
  // LDS read past a buffer store, so one read per store would serialise the round trips
  constexpr int G = 4;
  static_assert((WM / L::RPI) % G == 0, "read-back groups");
#pragma unroll
  for (int i0 = 0; i0 < WM / L::RPI; i0 += G) {
    i32x4 raw[G];
#pragma unroll
    for (int e = 0; e < G; ++e) {
      const int row = (i0 + e) * L::RPI + lane / L::LPR;
      raw[e] = *reinterpret_cast<const i32x4*>(scratch + row * L::RB + ((c ^ (L::swz(row) >> 1)) << 4));
    }
#pragma unroll
    for (int e = 0; e < G; ++e) {
      const int row = (i0 + e) * L::RPI + lane / L::LPR;
      const i32x4 v = (L::swz(row) & 1) ? i32x4{raw[e][2], raw[e][3], raw[e][0], raw[e][1]} : raw[e];
      const bool ok = cok && (m0w + row < M);
      const uint32_t off = ok ? (uint32_t)(((int64_t)row * N + 8 * c) * 2) : kOOB;
      __builtin_amdgcn_raw_buffer_store_b128(v, rd, off, 0, kStreamStore);
    }
  }
}

// Epilogue of one 32-row block b of a wave's tile through 32 rows of scratch
// (WN * 64 bytes), for kernels that keep the operand stages busy during the epilogue.
// The block is finished and staged as in epilogue_lds, then stored as whole row
// segments. `bv` is the bias of row 32 b + lane % 32 (unused by DRELU_BGRAD and NONE);
// for DRELU_BGRAD, mw[a] is the mask word of column n0w + 32 a + lane % 32 of the
// block's row group (0 outside the output).
// Consecutive calls may share the scratch: the stores of a block consume every value
// read back from it, so the next block's writes follow those reads.
template <int DT, int EP, int MB, int NB, int WN>
__device__ __forceinline__ void epilogue_block(const Args& p, const f32x16 (&acc)[NB][MB], int b, float bv,
                                               const uint32_t (&mw)[NB], int64_t m0w, int n0w, int lane,
                                               char* scratch) {
  using T = Tr<DT>;
  using L = EpiLayout<WN>;
  const int64_t M = p.m;
  const int N = p.n;
  const int lrow = lane & 31, lhi = lane >> 5;
  const int64_t mrow = m0w + 32 * b + lrow;
  const bool mok = mrow < M;
  const int64_t grp = (m0w + 32 * b) >> 5;
  const int s = L::swz(lrow);

  if constexpr (EP == DRELU_BGRAD) {
    float rowsum = 0.0f;
#pragma unroll
    for (int a = 0; a < NB; ++a) {
      const uint32_t word = mw[a];
      float dz[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        dz[r] = mask_bit_of_reg(word, r) ? acc[a][b][r] : 0.0f;
        rowsum += dz[r];
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int unit = (8 * a + 2 * g + lhi) ^ s;
        const i32x2 v = {(int)T::pack2(dz[4 * g], dz[4 * g + 1]), (int)T::pack2(dz[4 * g + 2], dz[4 * g + 3])};
        *reinterpret_cast<i32x2*>(scratch + lrow * L::RB + unit * 8) = v;
      }
    }
    rowsum += __shfl_xor(rowsum, 32);
    if (lhi == 0 && mok && n0w < N) p.partial[(int64_t)(n0w / WN) * M + mrow] = rowsum;
  } else {
#pragma unroll
    for (int a = 0; a < NB; ++a) {
      float pre[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) pre[r] = acc[a][b][r] + bv;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = activate<EP>(pre[4 * g + e]);
        const int unit = (8 * a + 2 * g + lhi) ^ s;
        const i32x2 v = {(int)T::pack2(y[0], y[1]), (int)T::pack2(y[2], y[3])};
        *reinterpret_cast<i32x2*>(scratch + lrow * L::RB + unit * 8) = v;
      }
      if constexpr (EP == RELU_AUX_BIAS) {
        const uint32_t word = relu_mask_words(pre, mok);
        const int ncol = n0w + 32 * a + lane;
        if (lane < 32 && grp * 32 < M && ncol < N) p.aux[grp * N + ncol] = word;
      }
    }
  }

  // all read-backs first, then the stores: the compiler does not move an LDS read
  // past a buffer store, so interleaving them would serialise the LDS round trips
  char* Dw = static_cast<char*>(p.D) + ((m0w + 32 * b) * (int64_t)N + n0w) * 2;
  const __amdgpu_buffer_rsrc_t rd = rsrc(Dw);
  const int c = lane % L::LPR;
  const bool cok = n0w + 8 * c < N;
  constexpr int NR = 32 / L::RPI;
  i32x4 raw[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const int row = i * L::RPI + lane / L::LPR;
    raw[i] = *reinterpret_cast<const i32x4*>(scratch + row * L::RB + ((c ^ (L::swz(row) >> 1)) << 4));
  }
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const int row = i * L::RPI + lane / L::LPR;
    const i32x4 v = (L::swz(row) & 1) ? i32x4{raw[i][2], raw[i][3], raw[i][0], raw[i][1]} : raw[i];
    const bool ok = cok && (m0w + 32 * b + row < M);
    const uint32_t off = ok ? (uint32_t)(((int64_t)row * N + 8 * c) * 2) : kOOB;
    __builtin_amdgcn_raw_buffer_store_b128(v, rd, off, 0, kStreamStore);
  }
}

// ---- operand copies and fragment reads shared by the main loops -----------------
template <int DT, int BM, int BN, int WM, int WN, int BK, int STAGES, int CW = 0>
struct Operands {
  using C = DtlCfg<BM, BN, WM, WN, BK, STAGES, CW>;
  static constexpr int MB = C::MB, NB = C::NB;
  static constexpr int A_PART = C::A_INST / C::KSTEPS, B_PART = C::B_INST / C::KSTEPS;

  const char* Abase;
  const char* Bbase;
  int N, K, w;
  uint32_t lds_base;
  uint32_t a_src[C::A_INST];
  int a_chunk[C::A_INST];
  uint32_t b_src[C::B_INST];
  int b_row[C::B_INST];
  int a_rd[C::KSTEPS];
  int b_rd[NB];

  __device__ __forceinline__ Operands(const Args& p, int64_t m0, int n0, int w_, int wm, int wn, int lane,
                                      uint32_t lds) {
    N = p.n;
    K = p.k;
    w = w_;
    lds_base = lds;
    retarget(p, m0, n0, lane);
    // fragment read addresses (stage-relative)
    const int lrow = lane & 31, lhi = lane >> 5;
#pragma unroll
    for (int s = 0; s < C::KSTEPS; ++s)
      a_rd[s] = (wm * WM + lrow) * C::A_ROWB + (((2 * s + lhi) ^ swz_a<C::A_ROWB>(lrow)) << 4);
    const int g = lane >> 4, i = lane & 15;
    const int row = 8 * lhi + (i >> 2);   // + 16 s (+ 4 for the second read)
#pragma unroll
    for (int a = 0; a < NB; ++a) {
      const int n = wn * WN + a * 32 + 16 * (g & 1) + 4 * (i & 3);
      b_rd[a] = C::A_BYTES + row * C::B_ROWB + (((n >> 3) ^ swz_b(row)) << 4) + ((n & 7) << 1);
    }
  }

  // Copy plan of the tile at (m0, n0): per-lane source offsets, constant over k.
  __device__ __forceinline__ void retarget(const Args& p, int64_t m0, int n0, int lane) {
    const int64_t M = p.m;
    Abase = static_cast<const char*>(p.A) + m0 * (int64_t)K * 2;
    Bbase = static_cast<const char*>(p.B) + (int64_t)n0 * 2;
#pragma unroll
    for (int j = 0; j < C::A_INST; ++j) {
      const int row = (w * C::A_INST + j) * C::A_RPI + lane / C::A_CHUNKS;
      const int c = (lane % C::A_CHUNKS) ^ swz_a<C::A_ROWB>(row);
      a_chunk[j] = c;
      a_src[j] = (m0 + row < M) ? (uint32_t)(row * K * 2 + c * 16) : kOOB;
    }
#pragma unroll
    for (int j = 0; j < C::B_INST; ++j) {
      const int row = (w * C::B_INST + j) * C::B_RPI + lane / C::B_CHUNKS;
      const int c = (lane % C::B_CHUNKS) ^ swz_b(row);
      b_row[j] = row;
      b_src[j] = (n0 + c * 8 < N) ? (uint32_t)(row * N * 2 + c * 16) : kOOB;
    }
  }

  // Copies A[a0, a1) and B[b0, b1) (instruction indices) of k-tile kt into LDS stage
  // `stage`.
  __device__ __forceinline__ void issue_range(int kt, int stage, int a0, int a1, int b0, int b1) const {
    const int k0 = kt * BK;
    const i32x4 ra = make_srd(Abase + (int64_t)k0 * 2);
    const i32x4 rb = make_srd(Bbase + (int64_t)k0 * N * 2);
    const uint32_t sA = lds_base + stage * C::STAGE;
    const uint32_t sB = sA + C::A_BYTES;
    const bool tail = k0 + BK > K;
#pragma unroll
    for (int j = 0; j < C::A_INST; ++j) {
      if (j < a0 || j >= a1) continue;
      const uint32_t off = (tail && k0 + a_chunk[j] * 8 >= K) ? kOOB : a_src[j];
      copy_to_lds_b128(ra, off, sA + (w * C::A_INST + j) * 1024);
    }
#pragma unroll
    for (int j = 0; j < C::B_INST; ++j) {
      if (j < b0 || j >= b1) continue;
      const uint32_t off = (tail && k0 + b_row[j] >= K) ? kOOB : b_src[j];
      copy_to_lds_b128(rb, off, sB + (w * C::B_INST + j) * 1024);
    }
  }
  // All copies of k-tile kt: in KSTEPS parts (A then B of each) when the counts divide,
  // else all A then all B.
  __device__ __forceinline__ void issue_tile(int kt, int stage) const {
    if constexpr (C::A_INST % C::KSTEPS == 0 && C::B_INST % C::KSTEPS == 0) {
#pragma unroll
      for (int part = 0; part < C::KSTEPS; ++part)
        issue_range(kt, stage, part * A_PART, (part + 1) * A_PART, part * B_PART, (part + 1) * B_PART);
    } else {
      issue_range(kt, stage, 0, C::A_INST, 0, C::B_INST);
    }
  }
};

// Fragments of one k-step read one instruction at a time, in the order the step's
// MFMAs consume them: B0 (two transposed halves), A0 .. A(MB-1), then B1 .. B(NB-1).
template <int MB, int NB>
struct Frags {
  static constexpr int PIECES = MB + 2 * NB;
  i32x4 a[MB];
  i32x2 b[NB][2];
  __device__ __forceinline__ i32x4 bfrag(int n) const { return i32x4{b[n][0][0], b[n][0][1], b[n][1][0], b[n][1][1]}; }
};

template <class O, int MB, int NB>
__device__ __forceinline__ void read_piece(const O& op, const char* base, int s, int q, Frags<MB, NB>& f) {
  constexpr int BROW = O::C::B_ROWB, AROW = O::C::A_ROWB;
  if (q < 2) {
    f.b[0][q] = ds_read_tr(base + op.b_rd[0] + 16 * s * BROW + q * 4 * BROW);
  } else if (q < 2 + MB) {
    f.a[q - 2] = *reinterpret_cast<const i32x4*>(base + op.a_rd[s] + (q - 2) * 32 * AROW);
  } else {
    const int n = (q - 2 - MB) / 2 + 1, h = (q - 2 - MB) % 2;
    f.b[n][h] = ds_read_tr(base + op.b_rd[n] + 16 * s * BROW + h * 4 * BROW);
  }
}

// ---- operands in either storage order ----------------------------------------------
// LAY bit 0: A is stored as A^T, a row-major (k, m) matrix; bit 1: B is stored as
// B^T, a row-major (n, k) matrix. An operand tile then sits in LDS in the order it
// has in memory:
//   k-major (A as stored normally, B given as B^T): MN rows of 2 BK bytes, 16-byte
//     chunks swizzled by swz_a, one ds_read_b128 per 32-row fragment (8 k values);
//   mn-major (B as stored normally, A given as A^T): BK rows of 2 MN bytes, chunks
//     swizzled by swz_b, two ds_read_b64_tr_b16 per fragment.
// Both give the MFMA operand layout (lane l: index l % 32 of the fragment's 32 rows or
// columns, k values 8 (l / 32) .. +7 of the k-step), so the main loop and epilogue
// do not depend on the layout.
template <int MN, int BK, bool KMAJ>
struct TileGeom {
  static constexpr int ROWB = KMAJ ? 2 * BK : 2 * MN;   // bytes per LDS row
  static constexpr int CHUNKS = ROWB / 16;
  static constexpr int RPI = 1024 / ROWB;               // rows per 1 KB copy instruction
  static_assert(KMAJ || MN >= 128, "mn-major rows hold at least 16 chunks");
  __device__ static __forceinline__ int swz(int row) {
    if constexpr (KMAJ) return swz_a<ROWB>(row);
    else return swz_b(row);
  }
};

// Copies of one operand's tile: INST 1 KB instructions per copying wave. The tile
// starts at row (k-major) or column (mn-major) mn0 of the stored matrix, whose
// extent along m or n is MNDIM; k runs over [0, K). Elements past MNDIM or K read
// as zero (out-of-range offsets).
template <int MN, int BK, bool KMAJ, int INST>
struct OperandCopy {
  using G = TileGeom<MN, BK, KMAJ>;
  const char* base;
  int64_t ldb;            // bytes between stored rows
  uint32_t src[INST];
  int kpos[INST];         // k offset inside the k-tile that decides the k tail

  __device__ __forceinline__ void init(const void* X, int64_t mn0, int64_t mndim, int K, int w, int lane) {
    if constexpr (KMAJ) {
      base = static_cast<const char*>(X) + mn0 * (int64_t)K * 2;
      ldb = (int64_t)K * 2;
    } else {
      base = static_cast<const char*>(X) + mn0 * 2;
      ldb = mndim * 2;
    }
#pragma unroll
    for (int j = 0; j < INST; ++j) {
      const int row = (w * INST + j) * G::RPI + lane / G::CHUNKS;
      const int c = (lane % G::CHUNKS) ^ G::swz(row);
      if constexpr (KMAJ) {
        kpos[j] = 8 * c;
        src[j] = (mn0 + row < mndim) ? (uint32_t)(row * ldb + c * 16) : kOOB;
      } else {
        kpos[j] = row;
        src[j] = (mn0 + 8 * c < mndim) ? (uint32_t)(row * ldb + c * 16) : kOOB;
      }
    }
  }
  // k-tile starting at k0 into the LDS region at `dst`.
  __device__ __forceinline__ void issue(int k0, int K, int w, uint32_t dst) const {
    const i32x4 srd = make_srd(base + (KMAJ ? (int64_t)k0 * 2 : (int64_t)k0 * ldb));
    const bool tail = k0 + BK > K;
#pragma unroll
    for (int j = 0; j < INST; ++j) {
      const uint32_t off = (tail && k0 + kpos[j] >= K) ? kOOB : src[j];
      copy_to_lds_b128(srd, off, dst + (w * INST + j) * 1024);
    }
  }
};

// Fragment reads of one operand for a wave whose fragments start at index wpos * W
// of the tile (NBLK fragments of 32, KS k-steps per k-tile), from the LDS region at
// byte `region` of a stage.
template <int MN, int BK, bool KMAJ, int W, int NBLK, int KS>
struct FragRead {
  using G = TileGeom<MN, BK, KMAJ>;
  int rd[KMAJ ? KS : NBLK];

  __device__ __forceinline__ void init(int wpos, int lane, int region) {
    const int lrow = lane & 31, lhi = lane >> 5;
    if constexpr (KMAJ) {
#pragma unroll
      for (int s = 0; s < KS; ++s)
        rd[s] = region + (wpos * W + lrow) * G::ROWB + (((2 * s + lhi) ^ G::swz(lrow)) << 4);
    } else {
      const int g = lane >> 4, i = lane & 15;
      const int row = 8 * lhi + (i >> 2);   // + 16 s, + 4 for the second read
#pragma unroll
      for (int blk = 0; blk < NBLK; ++blk) {
        const int x = wpos * W + blk * 32 + 16 * (g & 1) + 4 * (i & 3);
        rd[blk] = region + row * G::ROWB + (((x >> 3) ^ G::swz(row)) << 4) + ((x & 7) << 1);
      }
    }
  }
  __device__ __forceinline__ i32x4 read(const char* stage, int s, int blk) const {
    if constexpr (KMAJ) {
      return *reinterpret_cast<const i32x4*>(stage + rd[s] + blk * 32 * G::ROWB);
    } else {
      const char* q = stage + rd[blk] + 16 * s * G::ROWB;
      const i32x2 lo = ds_read_tr(q);
      const i32x2 hi = ds_read_tr(q + 4 * G::ROWB);
      return i32x4{lo[0], lo[1], hi[0], hi[1]};
    }
  }
  // mn-major only: half h (k values 4 h .. 4 h + 3 of the lane's eight) of a fragment
  __device__ __forceinline__ i32x2 read_half(const char* stage, int s, int blk, int h) const {
    static_assert(!KMAJ, "k-major fragments are one 16-byte read");
    return ds_read_tr(stage + rd[blk] + 16 * s * G::ROWB + h * 4 * G::ROWB);
  }
};

// Copies and fragment reads of both operands for LAY != 0 (the lockstep loop without
// interleaved reads or spread copies).
template <int DT, int BM, int BN, int WM, int WN, int BK, int STAGES, int CW, int LAY>
struct OperandsT {
  using C = DtlCfg<BM, BN, WM, WN, BK, STAGES, CW>;
  static constexpr bool TA = (LAY & 1) != 0, TB = (LAY & 2) != 0;
  static constexpr int MB = C::MB, NB = C::NB;
  OperandCopy<BM, BK, !TA, C::A_INST> ca;
  OperandCopy<BN, BK, TB, C::B_INST> cb;
  FragRead<BM, BK, !TA, WM, MB, C::KSTEPS> fa;
  FragRead<BN, BK, TB, WN, NB, C::KSTEPS> fb;
  int K, w;
  uint32_t lds_base;

  __device__ __forceinline__ OperandsT(const Args& p, int64_t m0, int n0, int w_, int wm, int wn, int lane,
                                       uint32_t lds) {
    K = p.k;
    w = w_;
    lds_base = lds;
    ca.init(p.A, m0, p.m, K, w, lane);
    cb.init(p.B, n0, p.n, K, w, lane);
    fa.init(wm, lane, 0);
    fb.init(wn, lane, C::A_BYTES);
  }
  __device__ __forceinline__ void issue_tile(int kt, int stage) const {
    const uint32_t sA = lds_base + stage * C::STAGE;
    ca.issue(kt * BK, K, w, sA);
    cb.issue(kt * BK, K, w, sA + C::A_BYTES);
  }
  // One instruction's worth of the fragments of k-step s, in the order the step's MFMAs
  // consume them: B block 0, the A blocks, then B blocks 1 .. NB-1; a k-major block is
  // one piece (ds_read_b128), an mn-major block two (its halves, ds_read_b64_tr_b16).
  static constexpr int PA = TA ? 2 : 1, PB = TB ? 1 : 2;
  static constexpr int PIECES = PB * NB + PA * MB;
  __device__ __forceinline__ void read_piece(const char* base, int s, int q, Frags<MB, NB>& f) const {
    int bq = q;   // piece index among the B pieces
    if (q >= PB) {
      if (q < PB + PA * MB) {
        const int blk = (q - PB) / PA;
        if constexpr (TA) {
          const i32x2 v = fa.read_half(base, s, blk, (q - PB) % PA);
          if ((q - PB) % PA == 0) {
            f.a[blk][0] = v[0];
            f.a[blk][1] = v[1];
          } else {
            f.a[blk][2] = v[0];
            f.a[blk][3] = v[1];
          }
        } else {
          f.a[blk] = fa.read(base, s, blk);
        }
        return;
      }
      bq = q - PA * MB;
    }
    const int blk = bq / PB;
    if constexpr (TB) {
      const i32x4 v = fb.read(base, s, blk);
      f.b[blk][0] = i32x2{v[0], v[1]};
      f.b[blk][1] = i32x2{v[2], v[3]};
    } else {
      f.b[blk][bq % PB] = fb.read_half(base, s, blk, bq % PB);
    }
  }

  // Every fragment of k-step s from the stage at `base`.
  __device__ __forceinline__ void read_step(const char* base, int s, Frags<MB, NB>& f) const {
#pragma unroll
    for (int b = 0; b < MB; ++b) f.a[b] = fa.read(base, s, b);
#pragma unroll
    for (int a = 0; a < NB; ++a) {
      const i32x4 v = fb.read(base, s, a);
      f.b[a][0] = i32x2{v[0], v[1]};
      f.b[a][1] = i32x2{v[2], v[3]};
    }
  }
};

// ---- lockstep main loop --------------------------------------------------------
// All waves run the same schedule. At the end of k-tile t every wave waits until
// its own copies of tile t+1 have landed and its reads of tile t are done, and one
// barrier publishes tile t+1 and releases stage t % STAGES.
// The copies of tile t + STAGES go to the released stage right after that barrier.
//   ILV = true:     each MFMA of a k-step is followed by one fragment read of the
//                   next step, in consumption order, instead of a block of reads.
//
// lockstep_tile accumulates the k-tiles [kb, kb + nt) of one output tile into acc.
// It expects no copy of its own in flight and every wave done with the LDS; on
// return every copy has landed, but reads of the last stage may still be in flight.
template <int DT, int BM, int BN, int WM, int WN, int BK, int STAGES, bool ILV, int CW, int LAY = 0>
__device__ __forceinline__ void lockstep_tile(const Args& p, char* smem, int64_t m0, int n0, int kb, int nt,
                                              f32x16 (&acc)[WN / 32][WM / 32]) {
  using C = DtlCfg<BM, BN, WM, WN, BK, STAGES, CW>;
  using O = std::conditional_t<LAY == 0, Operands<DT, BM, BN, WM, WN, BK, STAGES, CW>,
                               OperandsT<DT, BM, BN, WM, WN, BK, STAGES, CW, LAY>>;
  using F = Frags<C::MB, C::NB>;
  static_assert(DT == F16 || DT == BF16, "16-bit types only");
  static_assert(LAY == 0 || !ILV, "transposed operands use the plain lockstep loop");
  static_assert(C::KSTEPS % 2 == 0, "every tile starts on fragment buffer 0");
  constexpr int MB = C::MB, NB = C::NB, KS = C::KSTEPS;
  constexpr int NMMA = MB * NB;                          // MFMAs per k-step
  // interleaved reads: `PER` fragment reads after each MFMA (one unless a wave holds
  // more fragments than it issues MFMAs per k-step, as with three row blocks)
  constexpr int PER = (F::PIECES + NMMA - 1) / NMMA;

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = w % C::WAVES_M, wn = w / C::WAVES_M;
  const O op(p, m0, n0, w, wm, wn, lane, (uint32_t)(uintptr_t)(lds_void*)smem);
  const int KT = nt;   // k-tiles of this call; k-tile t is global k-tile kb + t
  const bool copier = w < C::CW;   // waves past CW issue no copies and wait for none

#pragma unroll
  for (int a = 0; a < NB; ++a)
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;
  F fr[2];

  auto read_all = [&](const char* base, int s, F& f) {
    if constexpr (LAY == 0) {
#pragma unroll
      for (int q = 0; q < F::PIECES; ++q) read_piece(op, base, s, q, f);
    } else {
      op.read_step(base, s, f);
    }
  };

  // prologue: tile 0 complete, the next tiles in flight
  if (copier) {
#pragma unroll
    for (int t = 0; t < STAGES; ++t)
      if (t < KT) op.issue_tile(kb + t, t);
    wait_tiles<C::INST, STAGES - 1>(min(STAGES - 1, KT - 1));
  }
  barrier_only();
  read_all(smem, 0, fr[0]);

  // Copies issued after tile kt+1's when tile kt reaches its barrier (the most there
  // can be in a steady tile).
  auto wait_next_tile = [&](int kt, auto steady_tag) {
    if constexpr (decltype(steady_tag)::value) {
      wait_vmcnt<(STAGES - 2) * C::INST>();
    } else {
      wait_tiles<C::INST, STAGES - 2>(min(STAGES - 2, KT - 2 - kt));
    }
  };

  // STEADY tiles (all but the last STAGES) read ahead and copy without checks, so the
  // MFMA stream carries no branches.
  auto tile = [&](auto steady_tag, int kt, int u) {
    constexpr bool STEADY = decltype(steady_tag)::value;
    const char* cur = smem + u * C::STAGE;
    const char* nxt = smem + ((u + 1) % STAGES) * C::STAGE;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int buf = s & 1;
      const bool last = s == KS - 1;
      if (last) {
        // the last step is in registers: publish tile kt+1 and release stage u
        wait_lgkmcnt<0>();                // this wave's reads of stage u are done
        if (copier) wait_next_tile(kt, steady_tag);   // this wave's copies of tile kt+1 have landed
        barrier_only();
        if (copier && (STEADY || kt + STAGES < KT)) op.issue_tile(kb + kt + STAGES, u);
      }
      const char* rbase = last ? nxt : cur;
      const int rs = last ? 0 : s + 1;
      const bool reads = STEADY || !last || kt + 1 < KT;
      if constexpr (!ILV) {
        if (reads) read_all(rbase, rs, fr[buf ^ 1]);
      }
#pragma unroll
      for (int i = 0; i < NMMA; ++i) {
        const int a = i / MB, b = i % MB;
        acc[a][b] = Tr<DT>::mma(fr[buf].bfrag(a), fr[buf].a[b], acc[a][b]);
        if constexpr (ILV) {
          if constexpr (LAY == 0) {
#pragma unroll
            for (int e = 0; e < PER; ++e) {
              const int q = i * PER + e;
              if (q < F::PIECES && reads) read_piece(op, rbase, rs, q, fr[buf ^ 1]);
            }
          }
        }
        if constexpr (ILV) __builtin_amdgcn_sched_barrier(0);
      }
      // keep each k-step's reads next to its MFMAs (no hoisting across steps)
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // A tile is steady when its reads of tile kt+1 and its copies of tile kt + STAGES
  // stay below KT.
  int kt = 0;
  for (; kt + 2 * STAGES <= KT; kt += STAGES) {
#pragma unroll
    for (int u = 0; u < STAGES; ++u) tile(std::true_type{}, kt + u, u);
  }
  for (; kt < KT; kt += STAGES) {
#pragma unroll
    for (int u = 0; u < STAGES; ++u)
      if (kt + u < KT) tile(std::false_type{}, kt + u, u);
  }
}

// One workgroup per output tile. LAY: storage order of the operands (OperandsT).
template <int DT, int EP, int BM, int BN, int WM, int WN, int BK, int STAGES, bool ILV, int CW, int LAY = 0>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64, 1) void gemm_dtl_kernel(Args p) {
  using C = DtlCfg<BM, BN, WM, WN, BK, STAGES>;
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS];
  int tm, tn;
  tile_coords(p, tm, tn);
  const int64_t m0 = (int64_t)tm * BM;
  const int n0 = tn * BN;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = w % C::WAVES_M, wn = w / C::WAVES_M;

  f32x16 acc[C::NB][C::MB];
  lockstep_tile<DT, BM, BN, WM, WN, BK, STAGES, ILV, CW, LAY>(p, smem, m0, n0, 0, (p.k + BK - 1) / BK, acc);

  // every wave is done with the stages: reuse them as per-wave epilogue scratch
  wait_lgkmcnt<0>();
  barrier_only();
  epilogue_lds<DT, EP, C::MB, C::NB, WN>(p, acc, m0 + wm * WM, n0 + wn * WN, lane, smem + w * C::SCRATCH);
}

// Operand copies of the persistent kernel, for K a multiple of BK. Each copy wave
// copies a contiguous block of rows of A (A_INST instructions of A_RPI rows) and of B
// (B_INST instructions of B_RPI k-rows). Per k-tile it builds one buffer descriptor per
// operand, with the k-tile and its row block in the base; an instruction's lanes take
// their offset inside the block from two per-parity lane offsets (the chunk swizzles
// repeat with the parity of the instruction) plus the instruction's row step, and its
// LDS slot from M0. Few scalar instructions per copy keep the copy waves close to the
// others at each k-tile's barrier.
template <int BM, int BN, int WM, int WN, int BK, int STAGES, int CW>
struct CopyPlan {
  using C = DtlCfg<BM, BN, WM, WN, BK, STAGES, CW>;
  static_assert(C::A_RPI % 8 == 0 || C::A_ROWB == 64, "A swizzle period");
  static_assert(C::B_RPI % 2 == 0, "B swizzle period");
  static_assert(C::A_INST % 2 == 0 && C::B_INST % 2 == 0, "copy parity follows j");

  const char* Arows;   // A at this wave's first copied row of the current tile, k = 0
  const char* Brows;   // B at this wave's first copied k-row, column n0 of the current tile
  uint32_t a_valid;    // bytes of this wave's copied rows of A that lie below m (rows * K * 2)
  int N, K, w;
  uint32_t lds_a, lds_b;           // this wave's first LDS copy slot of stage 0 (A, B)
  uint32_t a_lane[2], b_lane[2];   // lane offsets of an even / odd copy instruction
  uint32_t a_step, b_step;         // bytes between consecutive copy instructions

  __device__ __forceinline__ CopyPlan(const Args& p, int w_, int lane, uint32_t lds) {
    N = p.n;
    K = p.k;
    w = w_;
    lds_a = lds + w * C::A_INST * 1024;
    lds_b = lds + C::A_BYTES + w * C::B_INST * 1024;
    a_step = (uint32_t)(C::A_RPI * K * 2);
    b_step = (uint32_t)(C::B_RPI * N * 2);
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      const int row = par * C::A_RPI + lane / C::A_CHUNKS;
      const int c = (lane % C::A_CHUNKS) ^ swz_a<C::A_ROWB>(row);
      a_lane[par] = (uint32_t)((lane / C::A_CHUNKS) * K * 2 + c * 16);
    }
  }
  __device__ __forceinline__ void retarget(const Args& p, int64_t m0, int n0, int lane) {
    const int64_t r0 = m0 + (int64_t)w * C::A_INST * C::A_RPI;
    Arows = static_cast<const char*>(p.A) + r0 * (int64_t)K * 2;
    const int64_t rows = p.m - r0;
    a_valid = (uint32_t)((rows <= 0 ? 0 : rows >= C::A_INST * C::A_RPI ? C::A_INST * C::A_RPI : rows) * K * 2);
    Brows = static_cast<const char*>(p.B) + ((int64_t)w * C::B_INST * C::B_RPI * N + n0) * 2;
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      const int row = par * C::B_RPI + lane / C::B_CHUNKS;
      const int c = (lane % C::B_CHUNKS) ^ swz_b(row);
      b_lane[par] = (n0 + c * 8 < N) ? (uint32_t)((lane / C::B_CHUNKS) * N * 2 + c * 16) : kOOB;
    }
  }
  // One descriptor per operand and k-tile. A rows at or past m: the descriptor's range
  // ends at this wave's last valid row (every valid row's 128 bytes at k0 lie below it,
  // as k0 + BK <= K), so their offsets read as zero. B columns past n: kOOB lane offsets.
  __device__ __forceinline__ void issue_tile(int kt, int stage) const {
    const int64_t k0 = (int64_t)kt * BK;
    const uint32_t ka = (uint32_t)(k0 * 2);
    const i32x4 ra = make_srd(Arows + k0 * 2, a_valid > ka ? a_valid - ka : 0u);
    const i32x4 rb = make_srd(Brows + k0 * N * 2, 0x7fffffffu);
    const uint32_t sa = lds_a + stage * C::STAGE, sb = lds_b + stage * C::STAGE;
#pragma unroll
    for (int j = 0; j < C::A_INST; ++j)
      copy_to_lds_b128(ra, a_lane[j & 1] + j * a_step, sa + j * 1024);
#pragma unroll
    for (int j = 0; j < C::B_INST; ++j)
      copy_to_lds_b128(rb, b_lane[j & 1] + j * b_step, sb + j * 1024);
  }
};

// Copies of the persistent kernel for operands in either storage order (LAY != 0), on the
// pattern of CopyPlan: each copy wave copies a contiguous block of INST instructions of
// RPI stored rows; per k-tile one descriptor per operand, two per-parity lane offsets
// (the swizzle repeats with the parity of the instruction) plus the instruction's row
// step. K is a multiple of BK.
// k-major tile (A as stored, or B given as B^T): MN rows of 2 BK bytes; rows past the
// operand's extent fall outside the descriptor's range (which ends at this wave's last
// valid row; every valid row's 2 BK bytes at k0 lie below it) and read as zero.
template <int MN, int BK, int INST>
struct KMajorCopy {
  using G = TileGeom<MN, BK, true>;
  static_assert(G::RPI % 8 == 0 || G::ROWB == 64, "swizzle period");
  static_assert(INST % 2 == 0, "copy parity follows j");
  const char* rows;    // this wave's first copied row of the current tile, k = 0
  uint32_t valid;      // bytes of this wave's copied rows inside the extent
  uint32_t step;       // bytes between consecutive copy instructions (RPI rows)
  int64_t ldb;
  uint32_t lane_off[2];
  __device__ __forceinline__ void init(int K, int lane) {
    ldb = (int64_t)K * 2;
    step = (uint32_t)(G::RPI * ldb);
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      const int row = par * G::RPI + lane / G::CHUNKS;
      const int c = (lane % G::CHUNKS) ^ G::swz(row);
      lane_off[par] = (uint32_t)((lane / G::CHUNKS) * ldb + c * 16);
    }
  }
  __device__ __forceinline__ void retarget(const void* X, int64_t mn0, int64_t mndim, int w, int) {
    const int64_t r0 = mn0 + (int64_t)w * INST * G::RPI;
    rows = static_cast<const char*>(X) + r0 * ldb;
    const int64_t left = mndim - r0;
    valid = __builtin_amdgcn_readfirstlane(
        (int)((left <= 0 ? 0 : left >= INST * G::RPI ? INST * G::RPI : left) * ldb));
  }
  __device__ __forceinline__ void issue(int64_t k0, int w, uint32_t dst) const {
    const uint32_t kb = (uint32_t)(k0 * 2);
    const i32x4 srd = make_srd(rows + k0 * 2, valid > kb ? valid - kb : 0u);
    const uint32_t d = dst + w * INST * 1024;
#pragma unroll
    for (int j = 0; j < INST; ++j) copy_to_lds_b128(srd, lane_off[j & 1] + j * step, d + j * 1024);
  }
};
// mn-major tile (B as stored, or A given as A^T): BK rows of 2 MN bytes; columns past the
// operand's extent get an out-of-range lane offset.
template <int MN, int BK, int INST>
struct MNMajorCopy {
  using G = TileGeom<MN, BK, false>;
  static_assert(G::RPI % 2 == 0, "swizzle period");
  static_assert(INST % 2 == 0, "copy parity follows j");
  const char* rows;    // this wave's first copied k-row, column mn0 of the current tile
  uint32_t step;       // bytes between consecutive copy instructions (RPI k-rows)
  int64_t ldb;
  uint32_t lane_off[2];
  __device__ __forceinline__ void init(int, int) {}
  __device__ __forceinline__ void retarget(const void* X, int64_t mn0, int64_t mndim, int w, int lane) {
    ldb = mndim * 2;
    step = (uint32_t)(G::RPI * ldb);
    rows = static_cast<const char*>(X) + mn0 * 2 + (int64_t)w * INST * G::RPI * ldb;
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      const int row = par * G::RPI + lane / G::CHUNKS;
      const int c = (lane % G::CHUNKS) ^ G::swz(row);
      lane_off[par] = (mn0 + c * 8 < mndim) ? (uint32_t)((lane / G::CHUNKS) * ldb + c * 16) : kOOB;
    }
  }
  __device__ __forceinline__ void issue(int64_t k0, int w, uint32_t dst) const {
    const i32x4 srd = make_srd(rows + k0 * ldb, 0x7fffffffu);
    const uint32_t d = dst + w * INST * 1024;
#pragma unroll
    for (int j = 0; j < INST; ++j) copy_to_lds_b128(srd, lane_off[j & 1] + j * step, d + j * 1024);
  }
};

template <int BM, int BN, int WM, int WN, int BK, int STAGES, int CW, int LAY>
struct CopyPlanT {
  using C = DtlCfg<BM, BN, WM, WN, BK, STAGES, CW>;
  static constexpr bool TA = (LAY & 1) != 0, TB = (LAY & 2) != 0;
  std::conditional_t<TA, MNMajorCopy<BM, BK, C::A_INST>, KMajorCopy<BM, BK, C::A_INST>> ca;
  std::conditional_t<TB, KMajorCopy<BN, BK, C::B_INST>, MNMajorCopy<BN, BK, C::B_INST>> cb;
  int w;
  uint32_t lds_base;
  __device__ __forceinline__ CopyPlanT(const Args& p, int w_, int lane, uint32_t lds) {
    w = w_;
    lds_base = lds;
    ca.init(p.k, lane);
    cb.init(p.k, lane);
  }
  __device__ __forceinline__ void retarget(const Args& p, int64_t m0, int n0, int lane) {
    ca.retarget(p.A, m0, p.m, w, lane);
    cb.retarget(p.B, n0, p.n, w, lane);
  }
  __device__ __forceinline__ void issue_tile(int kt, int stage) const {
    const int64_t k0 = (int64_t)kt * BK;
    const uint32_t sA = lds_base + stage * C::STAGE;
    ca.issue(k0, w, sA);
    cb.issue(k0, w, sA + C::A_BYTES);
  }
};

// ---- persistent lockstep kernel --------------------------------------------------
// gridDim.x workgroups (one per compute unit) walk the tile order with that stride.
// The k loop runs on from one tile into the next: during a tile's last STAGES
// k-tiles the copy waves fetch the next tile's first STAGES k-tiles, so its operand
// latency hides behind the end of this tile and its epilogue. The epilogue works in
// 32-row blocks through LDS of its own (32 rows per wave), leaving the stages to
// those copies, and its stores drain while the next tile computes.
// Schedule per k-tile as in lockstep_tile with interleaved reads, plus: the first PRE
// MFMAs of a k-tile's last step are issued before its waits and barrier, so the
// matrix cores stay busy while the waves meet there. Every wave runs every vmcnt
// wait (the waves that copy nothing have only old stores and bias loads in flight),
// which also lets the compiler treat the bias loads as done by the epilogue.
// Requires K % BK == 0, KT % STAGES == 0 and KT >= 2 STAGES: k-tile t of every tile
// sits in stage t % STAGES.
// LAY != 0: operands in the storage orders of OperandsT (their fragment pieces) and
// CopyPlanT (their copies); the schedule is the same.
template <int DT, int EP, int BM, int BN, int WM, int WN, int BK, int STAGES, int CW, int PRE, int LAY = 0>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64, 1) void gemm_persist_kernel(Args p) {
  using C = DtlCfg<BM, BN, WM, WN, BK, STAGES, CW>;
  using O = std::conditional_t<LAY == 0, Operands<DT, BM, BN, WM, WN, BK, STAGES, CW>,
                               OperandsT<DT, BM, BN, WM, WN, BK, STAGES, CW, LAY>>;
  using CP = std::conditional_t<LAY == 0, CopyPlan<BM, BN, WM, WN, BK, STAGES, CW>,
                                CopyPlanT<BM, BN, WM, WN, BK, STAGES, CW, LAY>>;
  using F = Frags<C::MB, C::NB>;
  constexpr int MB = C::MB, NB = C::NB, KS = C::KSTEPS, NMMA = MB * NB;
  constexpr int PIECES = [] {
    if constexpr (LAY == 0) return F::PIECES;
    else return O::PIECES;
  }();
  constexpr int EPI_BYTES = 32 * WN * 2;   // epilogue rows of one wave
  static_assert(DT == F16 || DT == BF16, "16-bit types only");
  static_assert(C::LDS + C::NW * EPI_BYTES <= 160 * 1024, "LDS");
  static_assert(KS % 2 == 0, "every k-tile starts on fragment buffer 0");
  static_assert(PRE >= 0 && PRE < NMMA, "MFMA slots");
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS + C::NW * EPI_BYTES];

  const int T = p.tiles_m * p.tiles_n;
  const int KT = (p.k + BK - 1) / BK;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = w % C::WAVES_M, wn = w / C::WAVES_M;
  const bool copier = w < C::CW;
  char* scratch = smem + C::LDS + w * EPI_BYTES;

  int v = blockIdx.x;
  int tm, tn;
  raster(p, xcd_remap(v, T), tm, tn);
  int64_t m0 = (int64_t)tm * BM;
  int n0 = tn * BN;
  const uint32_t lds = (uint32_t)(uintptr_t)(lds_void*)smem;
  const O op(p, m0, n0, w, wm, wn, lane, lds);   // fragment reads only
  CP cp(p, w, lane, lds);
  cp.retarget(p, m0, n0, lane);
  auto piece = [&](const char* base, int s, int q, F& f) {
    if constexpr (LAY == 0) read_piece(op, base, s, q, f);
    else op.read_piece(base, s, q, f);
  };

  // Epilogue inputs, loaded when a tile starts and used in its epilogue (after the
  // k loop's vmcnt waits, so the epilogue never waits on the copies in flight then):
  // bias bits of rows 32 b + lane % 32 (converted in the epilogue), or for
  // DRELU_BGRAD the mask words of columns 32 a + lane % 32 of row group b.
  uint32_t bbits[MB];
  uint32_t mwords[MB][NB];
  auto load_bias = [&]() {
    const int l = opaque(lane);
#pragma unroll
    for (int b = 0; b < MB; ++b) {
      const int64_t row = m0 + wm * WM + 32 * b + (l & 31);
      bbits[b] = 0;
      if constexpr (EP != NONE && EP != DRELU_BGRAD) {
        if (row < p.m) bbits[b] = load_vec_bits(p.bias, p.vec_dt, row);
      }
      if constexpr (EP == DRELU_BGRAD) {
        const int64_t grp = (m0 + wm * WM + 32 * b) >> 5;
#pragma unroll
        for (int a = 0; a < NB; ++a) {
          const int ncol = n0 + wn * WN + 32 * a + (l & 31);
          mwords[b][a] = (grp * 32 < p.m && ncol < p.n) ? p.aux[grp * p.n + ncol] : 0u;
        }
      }
    }
  };
  // Each tile's first k-step gives its MFMAs a zero accumulator operand, so no
  // instruction clears the accumulators between tiles.
  f32x16 acc[NB][MB];
  F fr[2];
  auto read_all = [&](const char* base, int s, F& f) {
#pragma unroll
    for (int q = 0; q < PIECES; ++q) piece(base, s, q, f);
  };

  // One k-tile in stage u. NEXT = false: copies of this tile's k-tile kt + STAGES;
  // NEXT = true (the last STAGES k-tiles): copies of the next tile's k-tile
  // kt + STAGES - KT when there is a next tile, and no reads past the last k-tile.
  // FIRST = true: the tile's k-tile 0, whose first k-step starts from zero.
  auto ktile = [&](auto next_tag, auto first_tag, int kt, int u, bool more) {
    constexpr bool NEXT = decltype(next_tag)::value;
    constexpr bool FIRST = decltype(first_tag)::value;
    const char* cur = smem + u * C::STAGE;
    const char* nxt = smem + ((u + 1) % STAGES) * C::STAGE;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int buf = s & 1;
      const bool last = s == KS - 1;
      if (last) {
#pragma unroll
        for (int i = 0; i < PRE; ++i) {
          const int a = i / MB, b = i % MB;
          acc[a][b] = Tr<DT>::mma(fr[buf].bfrag(a), fr[buf].a[b], acc[a][b]);
        }
        __builtin_amdgcn_sched_barrier(0);
        // publish k-tile kt+1 (this tile's or the next tile's first) and release stage u
        wait_lgkmcnt<0>();
        if constexpr (NEXT) wait_tiles<C::INST, STAGES - 2>(more ? STAGES - 2 : min(STAGES - 2, KT - 2 - kt));
        else wait_vmcnt<(STAGES - 2) * C::INST>();
        barrier_only();
        if (copier) {
          if constexpr (NEXT) {
            if (more) cp.issue_tile(kt + STAGES - KT, u);
          } else {
            cp.issue_tile(kt + STAGES, u);
          }
        }
      }
      const char* rbase = last ? nxt : cur;
      const int rs = last ? 0 : s + 1;
      const bool reads = !NEXT || !last || kt + 1 < KT;
      const int i0 = last ? PRE : 0;
      const int per = (PIECES + NMMA - i0 - 1) / (NMMA - i0);
#pragma unroll
      for (int i = i0; i < NMMA; ++i) {
        const int a = i / MB, b = i % MB;
        acc[a][b] = Tr<DT>::mma(fr[buf].bfrag(a), fr[buf].a[b], FIRST && s == 0 ? f32x16{} : acc[a][b]);
#pragma unroll
        for (int e = 0; e < per; ++e) {
          const int q = (i - i0) * per + e;
          if (q < PIECES && reads) piece(rbase, rs, q, fr[buf ^ 1]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // prologue: the first tile's first STAGES k-tiles
  load_bias();
  if (copier) {
#pragma unroll
    for (int t = 0; t < STAGES; ++t) cp.issue_tile(t, t);
  }
  wait_vmcnt<0>();
  barrier_only();
  read_all(smem, 0, fr[0]);

  for (;;) {
    const int vn = v + (int)gridDim.x;
    const bool more = vn < T;
    int tmn = 0, tnn = 0;
    if (more) raster(p, xcd_remap(vn, T), tmn, tnn);
    // k-tiles 0 .. STAGES - 1 (KT >= 2 STAGES), then the rest up to the last STAGES
    ktile(std::false_type{}, std::true_type{}, 0, 0, more);
#pragma unroll
    for (int u = 1; u < STAGES; ++u) ktile(std::false_type{}, std::false_type{}, u, u, more);
    for (int kt = STAGES; kt < KT - STAGES; kt += STAGES) {
#pragma unroll
      for (int u = 0; u < STAGES; ++u) ktile(std::false_type{}, std::false_type{}, kt + u, u, more);
    }
    if (more) cp.retarget(p, (int64_t)tmn * BM, tnn * BN, opaque(lane));
#pragma unroll
    for (int u = 0; u < STAGES; ++u) ktile(std::true_type{}, std::false_type{}, KT - STAGES + u, u, more);

    const int elane = opaque(lane);   // the epilogue's lane arithmetic stays out of the k loop
#pragma unroll
    for (int b = 0; b < MB; ++b)
      epilogue_block<DT, EP, MB, NB, WN>(p, acc, b, vec_value(bbits[b], p.vec_dt), mwords[b], m0 + wm * WM,
                                         n0 + wn * WN, elane, scratch);
    if (!more) break;
    v = vn;
    m0 = (int64_t)tmn * BM;
    n0 = tnn * BN;
    load_bias();
    read_all(smem, 0, fr[0]);   // k-tile 0 of the new tile, published by the last barrier
  }
}

// ---- split tail of the tile grid -------------------------------------------------
// With T tiles on P compute units, T % P tiles would run as a last, partly empty
// round. gemm_sk_kernel runs dp_tiles = P * floor(T / P) tiles whole (one per
// workgroup, as gemm_dtl_kernel does) and hands the K loop of the remaining tiles to
// sk_wgs more workgroups, in equal runs of sk_units k-tiles taken in order over
// (tile, k-tile). Because sk_units < KT, a run holds at most one tile start: before
// it lies at most one piece that does not start at k = 0 (a partial), from it on the
// piece that does (the owner piece). The workgroup computes its partial first, stores
// it as fp32 in its slot and publishes it with the execute's epoch, then computes its
// owner piece, adds the partials of the runs that hold the rest of that tile and runs
// the epilogue. No workgroup waits before publishing its partial, so every wait ends
// once the workgroups it waits for have been scheduled. Runs are renumbered so each
// XCD takes a contiguous range of them.
//
// A partial slot holds, per wave, the fp32 accumulators as 4-float groups q, lane-
// minor (one 1 KB store per group). Partials cross XCDs, whose L2 caches are not
// coherent with each other: they are written and read with device-scope (sc1) buffer
// instructions, which write through to and read from the memory side, so publishing
// needs no writeback or invalidation of a whole L2.
template <int MB, int NB>
struct PartialLayout {
  static constexpr int QUADS = NB * MB * 4;                     // 4-float groups per lane
  static constexpr int WAVE_BYTES = QUADS * 64 * 16;
  __device__ static __forceinline__ uint32_t off(int w, int q, int lane) {
    return (uint32_t)(w * WAVE_BYTES + (q * 64 + lane) * 16);
  }
};
constexpr int kDeviceScope = 16;   // cache-policy bit sc1 of a buffer instruction

// Flag protocol of a published partial. A flag is 0 when idle. The run that computed
// the partial swaps 0 -> epoch once its stores have completed. The owner waits (a
// bounded spin, p.sk_spin_limit polls, about a second by default) for the epoch, adds
// the partial and swaps epoch -> 0. If the wait runs out, the owner swaps 0 -> kSkAbort
// (unless the epoch arrived meanwhile), counts the loss in p.sk_flag[kSkLostWord], gives
// the tile's D NaN; the publisher that finds kSkAbort resets the flag to 0 instead of
// publishing. So every flag is 0 again when the kernel ends, lost wait or not, and a
// later execute with the same epoch (a replay of a captured graph) never finds a stale
// one.
constexpr uint32_t kSkAbort = 0xffffffffu;   // epochs stay below 2^31

// Wave 0 of an owner waits for flags[0 .. np - 1], one lane per flag, so all the
// polls of one round trip are in flight together. Returns how many waits ran out
// (their flags now hold kSkAbort, or were published while the spin ran out).
__device__ __forceinline__ uint32_t sk_wait_flags(uint32_t* flags, int np, uint32_t epoch, uint32_t spin_limit,
                                                  int lane) {
  uint32_t lost = 0u;
  for (int j0 = 0; j0 < np; j0 += 64) {
    const int j = j0 + lane;
    uint32_t* f = flags + j;
    bool got = j >= np;
    for (uint32_t spins = 0; spins < spin_limit; ++spins) {
      if (!got) got = __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == epoch;
      if (__builtin_amdgcn_ballot_w64(!got) == 0) break;
      __builtin_amdgcn_s_sleep(2);
    }
    if (!got) {
      uint32_t expected = 0u;
      // abandoned: the late publisher will reset it; else published while the spin ran out
      if (!__hip_atomic_compare_exchange_strong(f, &expected, kSkAbort, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT))
        got = expected == epoch;
    }
    lost += (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(!got));
  }
  return lost;
}

// Split runs that cover whole tiles (KT a multiple of the run length): the S runs of
// tail tile t are t S .. t S + S - 1, run s computing k-tiles [s units, (s + 1) units).
// Workgroup q (each XCD takes a contiguous range of q) runs:
//   tiles of 256 rows, part-major: q = s T + t over the T tail tiles, so the runs that
//   share an XCD read A and B over the same k range, and tiles of one m-tile (n-tile)
//   share their A rows (B columns) in that XCD's L2 (2048 x 2048 x 8192: 3-5% faster
//   than tile-major);
//   smaller tiles (128 or 192 rows), tile-major: q = t S + s, so the S runs of a tile
//   share an XCD. The XCDs start a launch's workgroups up to about 2.5 us apart, and a
//   tile whose runs sit on several XCDs waits for the latest (1024 x 512 x 2048:
//   11.6 us tile-major, 14.3 part-major).
// The tile is finished in S parts, one per run: wave w's sub-tile belongs to run
// w % S. Every run stores the sub-tiles of its waves that other runs finish, publishes
// them, waits until all S runs have published, and its own waves add the other runs'
// partials of their sub-tiles (own sum first, then the others in run order) and run
// the epilogue. Each run thus moves (S - 1) / S of a tile each way instead of the
// owner's S - 1 tiles in one workgroup, and the epilogue is spread over S workgroups.
//
// Each tail tile has two counters in the flag region: words 2t (published) and 2t + 1
// (finished). A run adds 1 to the first once its stores have completed and waits (a
// bounded spin, p.sk_spin_limit polls) until it reads S; after its loads it adds 1 to
// the second, and the run that brings it to S sets both back to 0. Every run publishes
// before it waits and finishes after its wait, so the last to finish finds both
// complete and nothing touches them after it: the counters are 0 when the kernel ends,
// lost wait or not, and a replayed graph starts from clean counters. A wait that runs
// out is counted in the flag region's last word and gives NaN for the run's part.
template <int DT, int EP, int BM, int BN, int WM, int WN, int BK, int STAGES, bool ILV, int CW>
__device__ __forceinline__ void sk_reduce_scatter(const Args& p, char* smem, int q, int S, uint32_t& lost_any) {
  using C = DtlCfg<BM, BN, WM, WN, BK, STAGES>;
  using PL = PartialLayout<C::MB, C::NB>;
  constexpr int MB = C::MB, NB = C::NB;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = w % C::WAVES_M, wn = w / C::WAVES_M;
  const size_t slot_bytes = (size_t)C::NW * PL::WAVE_BYTES;
  const int T = p.sk_wgs / S;
  constexpr bool PART_MAJOR = BM >= 256;
  const int s = PART_MAJOR ? q / T : q % S;
  const int t = PART_MAJOR ? q - s * T : q / S;
  const int r = t * S + s;   // the run: its partial slot
  int tm, tn;
  raster(p, p.dp_tiles + t, tm, tn);

  f32x16 acc[NB][MB];
  lockstep_tile<DT, BM, BN, WM, WN, BK, STAGES, ILV, CW>(p, smem, (int64_t)tm * BM, tn * BN, s * p.sk_units,
                                                        p.sk_units, acc);
  const bool mine = w % S == s;
  char* const base = reinterpret_cast<char*>(p.sk_partial);
  if (!mine) {
    const __amdgpu_buffer_rsrc_t slot = rsrc(base + (size_t)r * slot_bytes);
#pragma unroll
    for (int a = 0; a < NB; ++a)
#pragma unroll
      for (int bb = 0; bb < MB; ++bb)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const i32x4 v = {__float_as_int(acc[a][bb][4 * r4]), __float_as_int(acc[a][bb][4 * r4 + 1]),
                           __float_as_int(acc[a][bb][4 * r4 + 2]), __float_as_int(acc[a][bb][4 * r4 + 3])};
          __builtin_amdgcn_raw_buffer_store_b128(v, slot, PL::off(w, (a * MB + bb) * 4 + r4, lane), 0, kDeviceScope);
        }
  }
  wait_vmcnt<0>();
  wait_lgkmcnt<0>();   // also: every wave is done with the LDS stages
  barrier_only();
  uint32_t* const cnt = p.sk_flag + 2 * t;   // [published, finished]
  // the epilogue's bias values (DRELU_BGRAD: mask words) load during the wait
  const int64_t m0w = (int64_t)tm * BM + wm * WM;
  const int n0w = tn * BN + wn * WN;
  uint32_t bbits[MB], mwords[MB][NB];
  if (mine) {
#pragma unroll
    for (int b = 0; b < MB; ++b) {
      const int64_t row = m0w + 32 * b + (lane & 31);
      bbits[b] = 0u;
      if constexpr (EP != NONE && EP != DRELU_BGRAD) {
        if (row < p.m) bbits[b] = load_vec_bits(p.bias, p.vec_dt, row);
      }
#pragma unroll
      for (int a = 0; a < NB; ++a) {
        mwords[b][a] = 0u;
        if constexpr (EP == DRELU_BGRAD) {
          const int64_t grp = (m0w + 32 * b) >> 5;
          const int ncol = n0w + 32 * a + (lane & 31);
          if (grp * 32 < p.m && ncol < p.n) mwords[b][a] = p.aux[grp * p.n + ncol];
        }
      }
    }
  }
  if (threadIdx.x == 0) {
    __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    bool all = false;
    for (uint32_t spins = 0; spins < p.sk_spin_limit && !all; ++spins) {
      all = __hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)S;
      if (!all) __builtin_amdgcn_s_sleep(2);
    }
    if (!all) all = __hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)S;
    if (!all) __hip_atomic_fetch_add(p.sk_flag + kSkLostWord, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    lost_any = all ? 0u : 1u;
  }
  wait_lgkmcnt<0>();
  barrier_only();
  const bool lost = lost_any != 0u;
  if (mine) {
    if (!lost) {
      // the other runs' partials of this sub-tile, read at device scope: LOADS loads in
      // flight at a time, QB 4-float groups of each of PB runs
      constexpr int LOADS = MB * NB <= 2 ? 24 : PL::QUADS % 16 == 0 ? 16 : 12;
      constexpr int QB = PL::QUADS < LOADS ? PL::QUADS : LOADS;
      constexpr int PB = LOADS / QB;
      static_assert(PL::QUADS % QB == 0, "load batches");
      for (int o0 = 0; o0 < S; o0 += PB) {
#pragma unroll
        for (int q0 = 0; q0 < PL::QUADS; q0 += QB) {
          i32x4 v[PB][QB];
#pragma unroll
          for (int i = 0; i < PB; ++i)
            if (o0 + i < S && o0 + i != s) {
              const __amdgpu_buffer_rsrc_t slot = rsrc(base + (size_t)(t * S + o0 + i) * slot_bytes);
#pragma unroll
              for (int j = 0; j < QB; ++j)
                v[i][j] = __builtin_amdgcn_raw_buffer_load_b128(slot, PL::off(w, q0 + j, lane), 0, kDeviceScope);
            }
#pragma unroll
          for (int i = 0; i < PB; ++i)
            if (o0 + i < S && o0 + i != s) {
#pragma unroll
              for (int j = 0; j < QB; ++j) {
                const int q = q0 + j, a = q / (4 * MB), bb = (q / 4) % MB, r4 = q % 4;
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[a][bb][4 * r4 + e] += __int_as_float(v[i][j][e]);
              }
            }
        }
      }
    } else {
#pragma unroll
      for (int a = 0; a < NB; ++a)
#pragma unroll
        for (int bb = 0; bb < MB; ++bb)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[a][bb][e] = __builtin_nanf("");
    }
  }
  // every wave's loads have completed before the run counts itself finished
  wait_vmcnt<0>();
  barrier_only();
  if (threadIdx.x == 0) {
    if (__hip_atomic_fetch_add(cnt + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(S - 1)) {
      __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(cnt + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (mine) {
#pragma unroll
    for (int b = 0; b < MB; ++b)
      epilogue_block<DT, EP, MB, NB, WN>(p, acc, b, vec_value(bbits[b], p.vec_dt), mwords[b], m0w, n0w, lane,
                                         smem + w * C::SCRATCH);
    // a lost wait: the activation may have turned the NaN accumulators into zeros, so
    // the sub-tile of D is written again with them as they are
    if (lost) {
#pragma unroll
      for (int b = 0; b < MB; ++b)
        epilogue_block<DT, NONE, MB, NB, WN>(p, acc, b, 0.0f, mwords[b], m0w, n0w, lane, smem + w * C::SCRATCH);
    }
  }
}

template <int DT, int EP, int BM, int BN, int WM, int WN, int BK, int STAGES, bool ILV, int CW>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64, 1) void gemm_sk_kernel(Args p) {
  using C = DtlCfg<BM, BN, WM, WN, BK, STAGES>;
  using PL = PartialLayout<C::MB, C::NB>;
  constexpr int MB = C::MB, NB = C::NB;
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = w % C::WAVES_M, wn = w / C::WAVES_M;
  const int KT = (p.k + BK - 1) / BK;
  const size_t slot_bytes = (size_t)C::NW * PL::WAVE_BYTES;

  // ---- this workgroup's pieces: a whole tile, or a run's partial and owner piece ----
  const bool split = (int)blockIdx.x >= p.dp_tiles;
  int r = 0;                                   // run
  SkRun run{0, 0, 0, 0, 0, 0};
  int pos, nt;                                 // whole tile or owner piece (nt == 0: none)
  if (!split) {
    pos = xcd_remap(blockIdx.x, p.dp_tiles);
    nt = KT;
  } else {
    r = xcd_remap(blockIdx.x - p.dp_tiles, p.sk_wgs);
    run = sk_run(r, p.sk_units, KT, p.tiles_m * p.tiles_n - p.dp_tiles, p.sk_wgs);
    pos = p.dp_tiles + run.own_t;
    nt = run.own_nt;
  }
  const int pa_t = run.pa_t, pa_kb = run.pa_kb, pa_nt = run.pa_nt;
  __shared__ uint32_t lost_any;

  if (split && KT % p.sk_units == 0) {
    sk_reduce_scatter<DT, EP, BM, BN, WM, WN, BK, STAGES, ILV, CW>(p, smem, r, KT / p.sk_units, lost_any);
    return;
  }

  f32x16 acc[NB][MB];
  bool lost = false;   // the owner: a partner's partial did not arrive in time
  if (pa_nt > 0) {
    int tm, tn;
    raster(p, p.dp_tiles + pa_t, tm, tn);
    lockstep_tile<DT, BM, BN, WM, WN, BK, STAGES, ILV, CW>(p, smem, (int64_t)tm * BM, tn * BN, pa_kb, pa_nt, acc);
    // store the partial at device scope, then publish it once every wave's stores
    // have completed
    const __amdgpu_buffer_rsrc_t slot = rsrc(reinterpret_cast<char*>(p.sk_partial) + (size_t)r * slot_bytes);
#pragma unroll
    for (int a = 0; a < NB; ++a)
#pragma unroll
      for (int bb = 0; bb < MB; ++bb)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const i32x4 v = {__float_as_int(acc[a][bb][4 * r4]), __float_as_int(acc[a][bb][4 * r4 + 1]),
                           __float_as_int(acc[a][bb][4 * r4 + 2]), __float_as_int(acc[a][bb][4 * r4 + 3])};
          __builtin_amdgcn_raw_buffer_store_b128(v, slot, PL::off(w, (a * MB + bb) * 4 + r4, lane), 0, kDeviceScope);
        }
    wait_vmcnt<0>();
    wait_lgkmcnt<0>();   // also: every wave is done with the LDS before the next piece
    barrier_only();
    if (threadIdx.x == 0) {
      uint32_t expected = 0u;
      if (!__hip_atomic_compare_exchange_strong(p.sk_flag + r, &expected, p.epoch, __ATOMIC_RELAXED,
                                                __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
        __hip_atomic_store(p.sk_flag + r, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);   // owner gave up
    }
  }
  if (nt == 0) return;

  int tm, tn;
  raster(p, pos, tm, tn);
  lockstep_tile<DT, BM, BN, WM, WN, BK, STAGES, ILV, CW>(p, smem, (int64_t)tm * BM, tn * BN, 0, nt, acc);
  if (split) {
    // the owner: wave 0 waits for the partials of runs r+1 .. last, which hold the rest
    // of the tile, and tells the workgroup through LDS whether all arrived
    if (w == 0) {
      const uint32_t lost = sk_wait_flags(p.sk_flag + r + 1, run.last - r, p.epoch, p.sk_spin_limit, lane);
      if (lane == 0) {
        if (lost) __hip_atomic_fetch_add(p.sk_flag + kSkLostWord, lost, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        lost_any = lost;
      }
    }
    wait_lgkmcnt<0>();
    barrier_only();
    // the partials' loads follow the flags seen before the barrier and read the memory
    // side (device scope)
    lost = lost_any != 0u;
    if (!lost) {
      // LOADS loads in flight at a time: QB 4-float groups of each of PB partials, then
      // the adds, partials in run order (the order of the sums does not depend on PB)
      constexpr int LOADS = MB * NB <= 2 ? 24 : PL::QUADS % 16 == 0 ? 16 : 12;
      constexpr int QB = PL::QUADS < LOADS ? PL::QUADS : LOADS;
      constexpr int PB = LOADS / QB;
      static_assert(PL::QUADS % QB == 0, "load batches");
      char* const base = reinterpret_cast<char*>(p.sk_partial);
      for (int o0 = r + 1; o0 <= run.last; o0 += PB) {
#pragma unroll
        for (int q0 = 0; q0 < PL::QUADS; q0 += QB) {
          i32x4 v[PB][QB];
#pragma unroll
          for (int i = 0; i < PB; ++i)
            if (o0 + i <= run.last) {
              const __amdgpu_buffer_rsrc_t slot = rsrc(base + (size_t)(o0 + i) * slot_bytes);
#pragma unroll
              for (int j = 0; j < QB; ++j)
                v[i][j] = __builtin_amdgcn_raw_buffer_load_b128(slot, PL::off(w, q0 + j, lane), 0, kDeviceScope);
            }
#pragma unroll
          for (int i = 0; i < PB; ++i)
            if (o0 + i <= run.last) {
#pragma unroll
              for (int j = 0; j < QB; ++j) {
                const int q = q0 + j, a = q / (4 * MB), bb = (q / 4) % MB, r4 = q % 4;
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[a][bb][4 * r4 + e] += __int_as_float(v[i][j][e]);
              }
            }
        }
      }
    } else {
#pragma unroll
      for (int a = 0; a < NB; ++a)
#pragma unroll
        for (int bb = 0; bb < MB; ++bb)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[a][bb][e] = __builtin_nanf("");
    }
  }
  // every wave is done with the stages: reuse them as per-wave epilogue scratch
  wait_vmcnt<0>();
  wait_lgkmcnt<0>();
  barrier_only();
  if (split && w == 0) {
    // every wave has read the partials: set the consumed flags (epoch) back to 0, one
    // lane per flag; an abandoned flag (kSkAbort) is reset by its late publisher
    for (int o = r + 1 + lane; o <= run.last; o += 64) {
      uint32_t expected = p.epoch;
      __hip_atomic_compare_exchange_strong(p.sk_flag + o, &expected, 0u, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  epilogue_lds<DT, EP, MB, NB, WN>(p, acc, (int64_t)tm * BM + wm * WM, tn * BN + wn * WN, lane,
                                   smem + w * C::SCRATCH);
  if (lost) {
    // the epilogue above wrote the mask (no bit set) and NaN row sums; an activation
    // may have turned the NaN accumulators into zeros, so D's tile is written again
    // with them as they are
    epilogue_lds<DT, NONE, MB, NB, WN>(p, acc, (int64_t)tm * BM + wm * WM, tn * BN + wn * WN, lane,
                                       smem + w * C::SCRATCH);
  }
}

}  // namespace gek
