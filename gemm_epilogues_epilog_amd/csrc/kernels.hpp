// Device code of the fused GEMM + epilogue library (gfx950 / CDNA4).
//
// One workgroup computes one BM x BN tile of D = epilogue(A . B):
//   * A (m,k) and B (k,n) are row-major. Each k-tile (128 bytes of k per row:
//     64 fp16/bf16 or 32 fp32 values) is staged through LDS in two buffers.
//     A rows are copied as 16-byte chunks; B is transposed in registers on its way
//     to LDS so both LDS tiles are "row = m or n, 128 bytes of k" with the 16-byte
//     chunks XOR-swizzled by row to keep the 64-lane fragment reads conflict-free.
//   * Each wave owns a WM x WN sub-tile built from 32x32 MFMA blocks with fp32
//     accumulators. The MFMA's row operand is the B^T fragment and its column
//     operand the A fragment, so in the accumulators lane l holds one row m of D
//     (l % 32) and its registers walk along n. This makes the ReLU mask a wavefront
//     ballot (32 rows of one column in one half of the ballot) and the bias
//     gradient an in-lane sum over registers plus one cross-half exchange.
//   * The epilogue (bias, activation, mask, masked gradient) runs on the
//     accumulators and D is written once.
//
// Method sources (web pages):
//  "Fusing bias addition via the nvmath-python epilog mechanism" (blog.hotdry.top),
//    paragraphs 2-3: bias of shape (m,1) added to every column; RELU_BIAS;
//    RELU_AUX_BIAS with a bit-encoded ReLU mask.
//  "nvmath-python wraps cuBLASLt" (blog.hotdry.top), body, plan step: FP32
//    accumulation for FP16 inputs and outputs; epilogue applied before the result
//    is written to memory.
//  "Fusing epilogs with matrix multiplication using nvmath-python" (itzkxy.com),
//    section "The DRELU_BGRAD path in the backward pass": mask applied to the product,
//    bias gradient returned as the sum over columns.
//  "Operator fusion in AI inference compilers" (mqxn.cn), section 2.2: the unfused
//    MatMul -> BiasAdd -> ReLU chain through two intermediate tensors.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gek {

enum Dt { F32 = 0, F16 = 1, BF16 = 2 };
enum Ep { NONE = 0, RELU_BIAS = 1, GELU_BIAS = 2, RELU_AUX_BIAS = 3, DRELU_BGRAD = 4, BIAS = 5 };

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// A buffer offset that is always outside the buffer: loads return 0, stores are dropped.
constexpr uint32_t kOOB = 0x80000000u;
constexpr int kRowBytes = 128;   // bytes of k per LDS row and per k-tile
constexpr int kBufDword3 = 0x00020000;

struct Args {
  const void* A;
  const void* B;
  const void* bias;
  void* D;
  uint32_t* aux;
  float* partial;     // DRELU_BGRAD: [ceil(n / WN)][m] per-wave row sums
  int64_t m;
  int32_t n;
  int32_t k;
  int32_t vec_dt;     // type of bias
  int32_t tiles_m;
  int32_t tiles_n;
  int32_t group_m;    // tile rasterisation: m-tiles per group
  // Split tail of the tile grid (direct-to-LDS kernels only; dp_tiles == all tiles
  // when unused): workgroups past the first dp_tiles share the remaining tiles'
  // k-tiles evenly, sk_units each.
  int32_t dp_tiles;   // tiles computed whole, one per workgroup
  int32_t sk_units;   // k-tiles per split workgroup
  int32_t sk_wgs;     // split workgroups
  uint32_t epoch;     // changes every execute; marks this execute's partials
  float* sk_partial;  // per split workgroup: one tile of fp32 partial accumulators
  uint32_t* sk_flag;  // per split workgroup: epoch of its published partial (and the
                      // count of owner waits that ran out at word kSkLostWord)
  uint32_t sk_spin_limit;   // polls of an owner's bounded wait for a partial
  // Persistent kernels: workgroups launched (one per compute unit), each walking the
  // tile order with that stride; 0 when the plan launches one workgroup per tile.
  int32_t persist_grid;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7fffffff, kBufDword3);
}

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding: vmcnt
// bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// s_waitcnt lgkmcnt(N) with the other counters left alone.
template <int N>
__device__ __forceinline__ void wait_lgkmcnt() {
  static_assert(N >= 0 && N < 16, "lgkmcnt range");
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (N << 8));
}

// v, through an empty volatile asm: the compiler cannot see that the result equals
// v, so values derived from it are computed where they are used instead of being
// hoisted out of a loop and kept live (or spilled) across it.
__device__ __forceinline__ int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Workgroup barrier that is also a compiler barrier for memory operations. It does
// not wait for outstanding memory operations: callers wait explicitly first.
__device__ __forceinline__ void barrier_only() { asm volatile("s_barrier" ::: "memory"); }

// Buffer descriptor (V#) as four SGPR values: base, no stride, `range` bytes (2^31 - 1
// by default), 32-bit data format. Offsets at or above kOOB are out of range.
__device__ __forceinline__ i32x4 make_srd(const void* base, uint32_t range = 0x7fffffffu) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane((int)range);
  r[3] = kBufDword3;
  return r;
}

// Direct global -> LDS copy of 16 bytes per lane: lane l reads srd.base + voff and
// writes LDS bytes [lds + 16 l, lds + 16 l + 16). Out-of-range offsets write zeros.
// Issued as inline assembly so that the compiler does not treat the copy as a write
// that every later LDS read must wait for; the caller orders it with wait_vmcnt and
// barrier_only. Loads complete in issue order, so the compiler's own vmcnt waits
// stay correct with these extra loads in flight (they can only wait longer). `lds`
// must be uniform; readfirstlane keeps it in an SGPR where the compiler cannot prove
// that by itself.
__device__ __forceinline__ void copy_to_lds_b128(const i32x4& srd, uint32_t voff, uint32_t lds) {
  // one wait state between the M0 write and the LDS-DMA load that reads it (gfx9)
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(srd), "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory", "m0");
}

// Workgroups are dealt to the 8 XCDs round-robin (id % 8). Renumber ids 0 .. G-1 so
// each XCD walks a contiguous range of positions.
__device__ __forceinline__ int xcd_remap(int id, int G) {
  const int per = G / 8, rem = G % 8, x = id % 8, local = id / 8;
  return (x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per) + local;
}

// Position in the tile order -> (m-tile, n-tile): groups of group_m m-tiles, m fastest
// inside a group, so tiles that run together share A and B in an XCD's L2.
__device__ __forceinline__ void raster(const Args& p, int pos, int& tm, int& tn) {
  const int gsz = p.group_m * p.tiles_n;
  const int g = pos / gsz, first_m = g * p.group_m;
  const int rows = min(p.tiles_m - first_m, p.group_m);
  const int in = pos - g * gsz;
  // the divisions run on the vector unit: pin the (uniform) results to SGPRs
  tm = __builtin_amdgcn_readfirstlane(first_m + in % rows);
  tn = __builtin_amdgcn_readfirstlane(in / rows);
}

// Workgroup id -> (m-tile, n-tile) when every workgroup computes one whole tile.
__device__ __forceinline__ void tile_coords(const Args& p, int& tm, int& tn) {
  raster(p, xcd_remap(blockIdx.x, p.tiles_m * p.tiles_n), tm, tn);
}

// ---- element traits ------------------------------------------------------------

template <int DT> struct Tr;

template <> struct Tr<F16> {
  static constexpr int es = 2;   // bytes per element
  static constexpr int E = 8;    // elements per 16-byte chunk
  // one k-step: 16 k values, two 16-byte chunks per row (one per half-wave)
  __device__ static __forceinline__ f32x16 mma(i32x4 a, i32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                  0, 0, 0);
  }
  // two values rounded to nearest even in one v_cvt_pk_f16_f32 (lo in bits 15:0)
  __device__ static __forceinline__ uint32_t pack2(float lo, float hi) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{lo, hi}), f16x2_t));
  }
  __device__ static __forceinline__ float widen(uint16_t v) { return (float)__builtin_bit_cast(_Float16, v); }
};

template <> struct Tr<BF16> {
  static constexpr int es = 2;
  static constexpr int E = 8;
  __device__ static __forceinline__ f32x16 mma(i32x4 a, i32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
  }
  // two values rounded to nearest even in one v_cvt_pk_bf16_f32 (lo in bits 15:0)
  __device__ static __forceinline__ uint32_t pack2(float lo, float hi) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{lo, hi}), bf16x2_t));
  }
  __device__ static __forceinline__ float widen(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }
};

template <> struct Tr<F32> {
  static constexpr int es = 4;
  static constexpr int E = 4;
  // one k-step: 8 k values; lane half h holds k = 4h + e of its chunk for MFMA e
  __device__ static __forceinline__ f32x16 mma(i32x4 a, i32x4 b, f32x16 c) {
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__int_as_float(a[0]), __int_as_float(b[0]), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__int_as_float(a[1]), __int_as_float(b[1]), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__int_as_float(a[2]), __int_as_float(b[2]), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__int_as_float(a[3]), __int_as_float(b[3]), c, 0, 0, 0);
    return c;
  }
};

// Element i of a bias vector as raw bits (fp32 bits, or the 16-bit value
// zero-extended), and their value: split so that a load can be issued long before
// its value is needed without the conversion forcing an early wait.
__device__ __forceinline__ uint32_t load_vec_bits(const void* p, int vec_dt, int64_t i) {
  if (vec_dt == F32) return static_cast<const uint32_t*>(p)[i];
  return static_cast<const uint16_t*>(p)[i];
}
__device__ __forceinline__ float vec_value(uint32_t bits, int vec_dt) {
  // selects, not branches: this sits between the blocks of an epilogue
  const float f = __uint_as_float(bits), h = Tr<F16>::widen((uint16_t)bits), g = Tr<BF16>::widen((uint16_t)bits);
  return vec_dt == F32 ? f : vec_dt == F16 ? h : g;
}

// ReLU mask words of one 32 x 32 accumulator block: lane c < 32 returns the word of
// block column c (bit i = pre of row i > 0; rows past m count as 0). Register r of
// lane l holds row l % 32 and column 8 (r / 4) + 4 (l / 32) + r % 4, so the ballot of
// register r holds column 8 (r / 4) + r % 4 in its low half and that column + 4 in
// its high half; each half is written straight into its column's lane.
// This lane's mask bit for register r: `word` holds in lane c (and c + 32) the mask
// word of block column c, and register r of lane l is row l % 32, column
// 8 (r / 4) + 4 (l / 32) + r % 4 of the block. Lanes 0-31 take their bits from the
// word of column c0 = 8 (r / 4) + r % 4 and lanes 32-63 from that of column c0 + 4, so
// the two words, read with readlane, form one 64-bit lane mask whose bit l is lane l's.
__device__ __forceinline__ bool mask_bit_of_reg(uint32_t word, int r) {
  const int c0 = 8 * (r >> 2) + (r & 3);
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readlane((int)word, c0);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readlane((int)word, c0 + 4);
  return __builtin_amdgcn_inverse_ballot_w64(hi << 32 | lo);
}

// Lane L of v = s (v_writelane_b32, immediate lane select). The compiler does not
// see into the asm, so it cannot space the instruction from a vector-ALU write of s
// (the ballot's compare): with WAIT, five wait states come first.
template <int L, bool WAIT>
__device__ __forceinline__ void write_lane(uint32_t& v, uint32_t s) {
  if constexpr (WAIT) asm("s_nop 4\n\tv_writelane_b32 %0, %1, %2" : "+v"(v) : "s"(s), "i"(L));
  else asm("v_writelane_b32 %0, %1, %2" : "+v"(v) : "s"(s), "i"(L));
}
template <int R = 0>
__device__ __forceinline__ void relu_mask_step(const float (&pre)[16], bool row_ok, uint32_t& word) {
  if constexpr (R < 16) {
    const uint64_t bal = __builtin_amdgcn_ballot_w64(row_ok && pre[R] > 0.0f);
    constexpr int cl = 8 * (R >> 2) + (R & 3);
    write_lane<cl, true>(word, (uint32_t)bal);
    write_lane<cl + 4, false>(word, (uint32_t)(bal >> 32));   // same producer, already spaced
    relu_mask_step<R + 1>(pre, row_ok, word);
  }
}
__device__ __forceinline__ uint32_t relu_mask_words(const float (&pre)[16], bool row_ok) {
  uint32_t word = 0;
  relu_mask_step(pre, row_ok, word);
  return word;
}

__device__ __forceinline__ float load_vec(const void* p, int vec_dt, int64_t i) {
  if (vec_dt == F32) return static_cast<const float*>(p)[i];
  const uint16_t v = static_cast<const uint16_t*>(p)[i];
  if (vec_dt == F16) return Tr<F16>::widen(v);
  return Tr<BF16>::widen(v);
}

__device__ __forceinline__ void store_vec(void* p, int vec_dt, int64_t i, float x) {
  if (vec_dt == F32) {
    static_cast<float*>(p)[i] = x;
  } else if (vec_dt == F16) {
    static_cast<_Float16*>(p)[i] = (_Float16)x;
  } else {
    static_cast<__bf16*>(p)[i] = (__bf16)x;
  }
}

// GELU, tanh form: 0.5 x (1 + tanh(u)) with u = sqrt(2/pi) (x + 0.044715 x^3).
// 0.5 (1 + tanh(u)) = 1 / (1 + 2^t) with t = -2 log2(e) u = x (c1 + c2 x^2), where
// c1 = -2 log2(e) sqrt(2/pi) and c2 = 0.044715 c1: one multiply, one fma and one
// multiply for t, then the hardware exp2 and reciprocal. 2^t overflowing to +inf
// gives x * 0 = 0, the correct limit.
__device__ __forceinline__ float gelu_tanh(float x) {
  constexpr float c1 = -2.302208198144325f;    // -2 log2(e) sqrt(2/pi)
  constexpr float c2 = -0.1029432395800235f;   // 0.044715 c1
  const float t = x * __builtin_fmaf(c2, x * x, c1);
  return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(t));
}

template <int EP>
__device__ __forceinline__ float activate(float pre) {
  if constexpr (EP == RELU_BIAS || EP == RELU_AUX_BIAS) return pre > 0.0f ? pre : 0.0f;
  else if constexpr (EP == GELU_BIAS) return gelu_tanh(pre);
  else return pre;
}

// ---- epilogue on the accumulators ---------------------------------------------
// A wave's accumulators acc[a][b] (32x32 MFMA blocks, fp32) cover rows m0w + 32 b
// and columns n0w + 32 a. Lane l holds row m0w + 32 b + l % 32; register r holds
// column n0w + 32 a + 8 (r / 4) + 4 (l / 32) + r % 4. D is written once, from here.
template <int DT, int EP, int MB, int NB, int WN>
__device__ __forceinline__ void epilogue(const Args& p, f32x16 (&acc)[NB][MB], int64_t m0w, int n0w, int lane) {
  using T = Tr<DT>;
  constexpr int es = T::es;
  const int64_t M = p.m;
  const int N = p.n;
  const int lrow = lane & 31, lhi = lane >> 5;
  char* Dw = static_cast<char*>(p.D) + (m0w * (int64_t)N + n0w) * es;
  const __amdgpu_buffer_rsrc_t rd = rsrc(Dw);

  if constexpr (EP == DRELU_BGRAD) {
#pragma unroll
    for (int b = 0; b < MB; ++b) {
      const int64_t mrow = m0w + 32 * b + lrow;
      const bool mok = mrow < M;
      const int64_t grp = (m0w + 32 * b) >> 5;
      const bool gok = grp * 32 < M;
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
          const int ncl = 32 * a + 8 * g + 4 * lhi;
          const bool ok = mok && (n0w + ncl < N);
          const uint32_t off = ok ? (uint32_t)(((32 * b + lrow) * (int64_t)N + ncl) * es) : kOOB;
          if constexpr (es == 2) {
            i32x2 v = {(int)T::pack2(dz[4 * g], dz[4 * g + 1]), (int)T::pack2(dz[4 * g + 2], dz[4 * g + 3])};
            __builtin_amdgcn_raw_buffer_store_b64(v, rd, off, 0, 0);
          } else {
            i32x4 v = {__float_as_int(dz[4 * g]), __float_as_int(dz[4 * g + 1]), __float_as_int(dz[4 * g + 2]),
                       __float_as_int(dz[4 * g + 3])};
            __builtin_amdgcn_raw_buffer_store_b128(v, rd, off, 0, 0);
          }
        }
      }
      rowsum += __shfl_xor(rowsum, 32);
      if (lhi == 0 && mok && n0w < N) p.partial[(int64_t)(n0w / WN) * M + mrow] = rowsum;
    }
  } else {
#pragma unroll
    for (int b = 0; b < MB; ++b) {
      const int64_t mrow = m0w + 32 * b + lrow;
      const bool mok = mrow < M;
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
          const int ncl = 32 * a + 8 * g + 4 * lhi;
          const bool ok = mok && (n0w + ncl < N);
          const uint32_t off = ok ? (uint32_t)(((32 * b + lrow) * (int64_t)N + ncl) * es) : kOOB;
          float y[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = activate<EP>(pre[4 * g + e]);
          if constexpr (es == 2) {
            i32x2 v = {(int)T::pack2(y[0], y[1]), (int)T::pack2(y[2], y[3])};
            __builtin_amdgcn_raw_buffer_store_b64(v, rd, off, 0, 0);
          } else {
            i32x4 v = {__float_as_int(y[0]), __float_as_int(y[1]), __float_as_int(y[2]), __float_as_int(y[3])};
            __builtin_amdgcn_raw_buffer_store_b128(v, rd, off, 0, 0);
          }
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
}
// ---- unfused baseline, kernels 2 and 3 ----------------------------------------
// T2 = round(T1 + bias[row]) and D = max(T2, 0), 16 bytes per thread, rows of n
// elements (n is a multiple of the 16-byte element count).
template <int DT>
__global__ __launch_bounds__(256) void bias_add_kernel(const void* __restrict__ in, const void* __restrict__ bias,
                                                       int vec_dt, void* __restrict__ out, int64_t chunks, int n) {
  constexpr int E = Tr<DT>::E;
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= chunks) return;
  const int64_t row = (c * E) / n;
  const float bv = load_vec(bias, vec_dt, row);
  const i32x4 v = static_cast<const i32x4*>(in)[c];
  i32x4 o;
  if constexpr (DT == F32) {
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = __float_as_int(__int_as_float(v[e]) + bv);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t u = (uint32_t)v[e];
      const float lo = Tr<DT>::widen((uint16_t)(u & 0xffffu)) + bv;
      const float hi = Tr<DT>::widen((uint16_t)(u >> 16)) + bv;
      o[e] = (int)Tr<DT>::pack2(lo, hi);
    }
  }
  static_cast<i32x4*>(out)[c] = o;
}

template <int DT>
__global__ __launch_bounds__(256) void relu_kernel(const void* __restrict__ in, void* __restrict__ out,
                                                   int64_t chunks) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= chunks) return;
  const i32x4 v = static_cast<const i32x4*>(in)[c];
  i32x4 o;
  if constexpr (DT == F32) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x = __int_as_float(v[e]);
      o[e] = __float_as_int(x > 0.0f ? x : 0.0f);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t u = (uint32_t)v[e];
      const float lo = Tr<DT>::widen((uint16_t)(u & 0xffffu));
      const float hi = Tr<DT>::widen((uint16_t)(u >> 16));
      o[e] = (int)Tr<DT>::pack2(lo > 0.0f ? lo : 0.0f, hi > 0.0f ? hi : 0.0f);
    }
  }
  static_cast<i32x4*>(out)[c] = o;
}

// ---- unfused backward baseline, kernels 2 and 3 ---------------------------------
// D = T1 where the forward activation is > 0, else +0 (the ReLU backward as its own
// kernel, reading the activation the unfused forward stored), 16 bytes per thread.
template <int DT>
__global__ __launch_bounds__(256) void drelu_kernel(const void* __restrict__ in, const void* __restrict__ act,
                                                    void* __restrict__ out, int64_t chunks) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= chunks) return;
  const i32x4 v = static_cast<const i32x4*>(in)[c];
  const i32x4 a = static_cast<const i32x4*>(act)[c];
  i32x4 o;
  if constexpr (DT == F32) {
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = __int_as_float(a[e]) > 0.0f ? v[e] : 0;
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t u = (uint32_t)a[e];
      const uint32_t keep_lo = Tr<DT>::widen((uint16_t)(u & 0xffffu)) > 0.0f ? 0x0000ffffu : 0u;
      const uint32_t keep_hi = Tr<DT>::widen((uint16_t)(u >> 16)) > 0.0f ? 0xffff0000u : 0u;
      o[e] = (int)((uint32_t)v[e] & (keep_lo | keep_hi));
    }
  }
  static_cast<i32x4*>(out)[c] = o;
}

// bgrad[row] = the sum of the row's n stored values, one wave per row: lane l adds the
// 16-byte chunks l, l + 64, l + 128, ... in ascending order (kRowSumBatch loads in
// flight), then the lanes' sums are added by a fixed butterfly, so results repeat bit
// for bit.
constexpr int kRowSumBatch = 4;
template <int DT>
__global__ __launch_bounds__(256) void row_sum_kernel(const void* __restrict__ in, int64_t m, int n,
                                                      void* __restrict__ bgrad, int vec_dt) {
  constexpr int E = Tr<DT>::E;
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= m) return;
  const int chunks = n / E;
  const i32x4* p = static_cast<const i32x4*>(in) + row * chunks;
  float s = 0.0f;
  for (int c0 = lane; c0 < chunks; c0 += 64 * kRowSumBatch) {
    i32x4 v[kRowSumBatch];
#pragma unroll
    for (int u = 0; u < kRowSumBatch; ++u) {
      const int c = c0 + 64 * u;
      v[u] = c < chunks ? p[c] : i32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kRowSumBatch; ++u) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (DT == F32) {
          s += __int_as_float(v[u][e]);
        } else {
          const uint32_t w = (uint32_t)v[u][e];
          s += Tr<DT>::widen((uint16_t)(w & 0xffffu));
          s += Tr<DT>::widen((uint16_t)(w >> 16));
        }
      }
    }
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) s += __shfl_xor(s, off);
  if (lane == 0) store_vec(bgrad, vec_dt, row, s);
}

}  // namespace gek
