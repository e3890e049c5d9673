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
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7fffffff, kBufDword3);
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
  __device__ static __forceinline__ uint32_t pack2(float lo, float hi) {
    const uint32_t l = __builtin_bit_cast(uint16_t, (_Float16)lo);
    const uint32_t h = __builtin_bit_cast(uint16_t, (_Float16)hi);
    return l | (h << 16);
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
  __device__ static __forceinline__ uint32_t pack2(float lo, float hi) {
    const uint32_t l = __builtin_bit_cast(uint16_t, (__bf16)lo);
    const uint32_t h = __builtin_bit_cast(uint16_t, (__bf16)hi);
    return l | (h << 16);
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
// 0.5 (1 + tanh(u)) = 1 / (1 + e^{-2u}), evaluated with the hardware exp2 and
// reciprocal. e^{-2u} overflowing to +inf gives x * 0 = 0, the correct limit.
__device__ __forceinline__ float gelu_tanh(float x) {
  const float u = 0.7978845608028654f * (x + 0.044715f * x * x * x);
  const float e = __builtin_amdgcn_exp2f(-2.8853900817779268f * u);   // -2 log2(e) u
  return x * __builtin_amdgcn_rcpf(1.0f + e);
}

template <int EP>
__device__ __forceinline__ float activate(float pre) {
  if constexpr (EP == RELU_BIAS || EP == RELU_AUX_BIAS) return pre > 0.0f ? pre : 0.0f;
  else if constexpr (EP == GELU_BIAS) return gelu_tanh(pre);
  else return pre;
}

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

  // ---- tile rasterisation ----------------------------------------------------
  // Workgroups are dealt to the 8 XCDs round-robin; renumber them so that each XCD
  // walks a contiguous range of tiles, then walk tiles in groups of group_m m-tiles
  // (m fastest inside a group) so tiles running together share A and B in L2.
  const int G = p.tiles_m * p.tiles_n;
  int id = blockIdx.x;
  {
    const int per = G / 8, rem = G % 8, x = id % 8, local = id / 8;
    id = (x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per) + local;
  }
  int tm, tn;
  {
    const int gsz = p.group_m * p.tiles_n;
    const int g = id / gsz, first_m = g * p.group_m;
    const int rows = min(p.tiles_m - first_m, p.group_m);
    const int in = id - g * gsz;
    tm = first_m + in % rows;
    tn = in / rows;
  }
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

  // ---- epilogue on the accumulators ------------------------------------------
  // acc[a][b][r]: row m = m0w + 32 b + lrow, column n = n0w + 32 a + 8 (r/4) + 4 lhi + r%4
  const int64_t m0w = m0 + wm * WM;
  const int n0w = n0 + wn * WN;
  char* Dw = static_cast<char*>(p.D) + (m0w * (int64_t)N + n0w) * es;
  const __amdgpu_buffer_rsrc_t rd = rsrc(Dw);

  if constexpr (EP == DRELU_BGRAD) {
    const uint32_t mybit = 1u << lrow;
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
          const int idx = 8 * (r >> 2) + (r & 3);
          const uint32_t wl = __builtin_amdgcn_readlane(word, idx);
          const uint32_t wh = __builtin_amdgcn_readlane(word, idx + 4);
          const uint32_t wr = lhi ? wh : wl;
          dz[r] = (wr & mybit) ? acc[a][b][r] : 0.0f;
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
          // ballot r: bits 0-31 = rows of column 8(r/4) + r%4, bits 32-63 = column +4
          uint32_t word = 0;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const uint64_t bal = __ballot(mok && pre[r] > 0.0f);
            const int cl = 8 * (r >> 2) + (r & 3);
            if (lane == cl) word = (uint32_t)bal;
            if (lane == cl + 4) word = (uint32_t)(bal >> 32);
          }
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

}  // namespace gek
