// CPU oracle for the fused GEMM-epilogue path.
//
// TEST INFRASTRUCTURE ONLY. Nothing in the product path may call, link or load
// this file; only the test-suite, the smoke check and the benchmark's CPU-baseline
// leg do. It shares no code, header, table or helper with the HIP library.
//
// What it computes is the plain definition of each epilogue, element by element:
//
//   acc[i,j] = sum_{kk ascending} fl32(a[i,kk] * b[kk,j])        fp32 accumulator
//   pre[i,j] = fl32(acc[i,j] + bias[i])                          bias along rows
//   D[i,j]   = round_to_nearest_even_d( act(pre[i,j]) )
//
// Sources (the web pages this method is described on):
//  * "Fusing bias addition via the nvmath-python epilog mechanism: parameter
//    configuration and engineering practice guide" (blog.hotdry.top), paragraph 2:
//    the BIAS epilog takes a bias of shape (m,) or (m,1) and adds it to every
//    column of the (m,n) product; paragraph 3: RELU_BIAS applies ReLU after the
//    bias, RELU_AUX_BIAS also returns a bit-encoded ReLU mask for the backward pass.
//  * "nvmath-python wraps cuBLASLt: low-overhead matmul and bias-fusion primitives
//    for PyTorch" (blog.hotdry.top), body, plan step: the compute type keeps FP16
//    inputs and outputs with an FP32 accumulator; the "other epilogs" paragraph
//    names BIAS, GELU_BIAS and RELU_AUX_BIAS.
//  * "Fusing epilogs with matrix multiplication using nvmath-python" (itzkxy.com),
//    section "The DRELU_BGRAD path in the backward pass": the stored ReLU mask is
//    applied to the matmul result and the bias gradient is returned as a sum over
//    the columns of every row.
//  * "Operator fusion in AI inference compilers: implementation and trade-offs"
//    (mqxn.cn), section 2.2 diagram: the unfused chain MatMul -> T1 -> BiasAdd ->
//    T2 -> ReLU, each operator its own kernel with its output written to memory;
//    section 2.3 / 4.3: fusion must give the same result up to the order of the
//    floating-point reduction, with FP32 accumulation.
//
// Readings where the pages are silent (each is also listed with the design notes):
//  * mask layout: uint32 words [ceil(m/32)][n]; bit (i % 32) of word (i/32, j) is
//    1 exactly when pre[i,j] > 0 (strict); bits for rows i >= m are 0.
//  * ReLU of pre <= 0 (and of NaN) is +0.0; dReLU uses the same strict test.
//  * GELU is the tanh form 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))),
//    evaluated in double from the fp32 pre-activation, then rounded to fp32 and
//    then to D's type.
//  * DRELU_BGRAD: dz = bit ? acc : +0; D = round(dz); bgrad[i] = round_vec(sum_j
//    dz[i,j]) with the sum taken in double over ascending j.
//  * unfused chain: T1 = round_d(acc); T2 = round_d(T1 + bias); D = max(T2, 0).
//  * unfused backward chain (the three steps DRELU_BGRAD does in one call, each as its
//    own kernel as in the diagram above): T1 = round_d(acc); D = act > 0 ? T1 : +0,
//    where act is the forward pass's stored activation (D's type; the unfused forward
//    keeps its ReLU output, not a bit mask); bgrad[i] = round_vec(sum_j D[i,j]) with
//    the sum of the stored D values taken in double over ascending j.
//
// Operand storage order ("Fusing epilogs with matrix multiplication using
// nvmath-python", section on the DRELU_BGRAD path, second paragraph: the backward's
// weight transpose must match the matmul call): with trans_a the A argument holds the
// row-major (k, m) matrix At and a[i,kk] = At[kk,i]; with trans_b the B argument holds
// the row-major (n, k) matrix Bt and b[kk,j] = Bt[j,kk]. The product is the same sum.
//
// Special values: infinities and NaN in the operands propagate through the products and
// sums as IEEE arithmetic gives them, ReLU of NaN is +0 with mask bit 0, and D's rounding
// overflows to +-inf (fp16: from the tie at 65520 on); pinned against float64 elementwise
// products in the tests. The sign of zero at the ReLU tie is pinned as well.
//
// Build: g++ -O3 -march=x86-64-v3 -ffp-contract=off -fno-fast-math -shared -fPIC -pthread
// -ffp-contract=off keeps every product and every sum individually rounded.

#include <cmath>
#include <cstdint>
#include <cstring>
#include <cstdlib>
#include <thread>
#include <vector>
#include <algorithm>

namespace {

// dtype codes of this file's C interface (chosen to match the library's public enum).
enum { ODT_F32 = 0, ODT_F16 = 1, ODT_BF16 = 2 };
// epilogue codes of this file's C interface (chosen to match the library's public enum).
enum { OEP_NONE = 0, OEP_RELU_BIAS = 1, OEP_GELU_BIAS = 2, OEP_RELU_AUX_BIAS = 3,
       OEP_DRELU_BGRAD = 4, OEP_BIAS = 5, OEP_RELU_BIAS_UNFUSED = 100, OEP_DRELU_BGRAD_UNFUSED = 101 };

inline uint32_t f32_bits(float x) { uint32_t u; std::memcpy(&u, &x, 4); return u; }
inline float bits_f32(uint32_t u) { float x; std::memcpy(&x, &u, 4); return x; }

// ---- IEEE binary16 <-> binary32 -------------------------------------------------

// Exact widening of a binary16 pattern.
float f16_to_f32(uint16_t h) {
  uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
  uint32_t e = (h >> 10) & 0x1fu;
  uint32_t f = h & 0x3ffu;
  if (e == 0x1f) return bits_f32(sign | 0x7f800000u | (f << 13));       // inf / NaN
  if (e == 0) {
    // zero or subnormal: value = f * 2^-24, exact in binary32
    float v = (float)f * 5.9604644775390625e-8f;
    return sign ? -v : v;
  }
  return bits_f32(sign | ((e + 112u) << 23) | (f << 13));
}

// binary32 -> binary16, round to nearest, ties to even. Overflow gives +-inf,
// subnormal results are kept, NaN becomes a quiet NaN.
uint16_t f32_to_f16(float x) {
  uint32_t u = f32_bits(x);
  uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
  uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return sign | 0x7e00u;             // NaN
  if (a >= 0x477ff000u) return sign | 0x7c00u;            // |x| >= 65520 -> inf
  if (a >= 0x38800000u) {                                 // result is a normal half
    uint32_t r = a + 0xfffu + ((a >> 13) & 1u);           // RNE at bit 13
    return sign | (uint16_t)((r - (112u << 23)) >> 13);
  }
  // result is subnormal or zero: count units of 2^-24, rounding to nearest even
  float q = bits_f32(a) * 16777216.0f;                    // exact scaling by 2^24
  float qi = std::nearbyint(q);                           // default mode: ties to even
  return sign | (uint16_t)qi;
}

// ---- bfloat16 <-> binary32 -------------------------------------------------------

float bf16_to_f32(uint16_t h) { return bits_f32((uint32_t)h << 16); }

uint16_t f32_to_bf16(float x) {
  uint32_t u = f32_bits(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);   // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);                                                // RNE
  return (uint16_t)(u >> 16);
}

float load_elem(const void* p, int dt, int64_t idx) {
  switch (dt) {
    case ODT_F32: return static_cast<const float*>(p)[idx];
    case ODT_F16: return f16_to_f32(static_cast<const uint16_t*>(p)[idx]);
    default:      return bf16_to_f32(static_cast<const uint16_t*>(p)[idx]);
  }
}

void store_elem(void* p, int dt, int64_t idx, float v) {
  switch (dt) {
    case ODT_F32: static_cast<float*>(p)[idx] = v; break;
    case ODT_F16: static_cast<uint16_t*>(p)[idx] = f32_to_f16(v); break;
    default:      static_cast<uint16_t*>(p)[idx] = f32_to_bf16(v); break;
  }
}

// Round a float to the precision of dtype dt and back (value as stored, then re-read).
float round_through(int dt, float v) {
  switch (dt) {
    case ODT_F32: return v;
    case ODT_F16: return f16_to_f32(f32_to_f16(v));
    default:      return bf16_to_f32(f32_to_bf16(v));
  }
}

double gelu_tanh(double x) {
  const double c = 0.7978845608028654;   // sqrt(2/pi)
  return 0.5 * x * (1.0 + std::tanh(c * (x + 0.044715 * x * x * x)));
}

float relu(float p) { return p > 0.0f ? p : 0.0f; }

struct Problem {
  int64_t m, n, k;
  int ab_dt, d_dt, vec_dt, epilog;
  const float* Aw;        // widened A, m x k
  const float* Bw;        // widened B, k x n
  const void* bias;       // m values in vec_dt (forward epilogs with a bias)
  void* D;                // m x n in d_dt
  uint32_t* aux;          // mask words: written for RELU_AUX_BIAS, read for DRELU_BGRAD
  void* bgrad;            // m values in vec_dt (DRELU_BGRAD, DRELU_BGRAD_UNFUSED)
  const void* act;        // m x n in d_dt: the forward activation (DRELU_BGRAD_UNFUSED)
  float* pre_out;         // optional m x n: pre-activation (or dz for the backward)
  double* absum_out;      // optional m: sum_j |dz[i,j]| (the backward)
};

// Rows [r0, r1) of the result. r0 is a multiple of 32 so mask words are owned by
// exactly one worker.
void compute_rows(const Problem& P, int64_t r0, int64_t r1) {
  const int64_t n = P.n, k = P.k;
  const int64_t RB = 32;                 // rows that share each row of B
  const int64_t JB = 256;                // columns whose accumulators stay in cache
  std::vector<float> acc((size_t)(RB * JB));
  std::vector<double> rowsum((size_t)RB), rowabs((size_t)RB);

  for (int64_t i0 = r0; i0 < r1; i0 += RB) {
    const int64_t ib = std::min(RB, r1 - i0);
    std::fill(rowsum.begin(), rowsum.end(), 0.0);
    std::fill(rowabs.begin(), rowabs.end(), 0.0);
    if (P.epilog == OEP_RELU_AUX_BIAS) {
      // clear the words of this row group (all 32 rows belong to this block)
      uint32_t* w = P.aux + (i0 / 32) * n;
      std::fill(w, w + n, 0u);
    }
    for (int64_t j0 = 0; j0 < n; j0 += JB) {
      const int64_t jb = std::min(JB, n - j0);
      std::fill(acc.begin(), acc.end(), 0.0f);
      // product sum, ascending kk for every element
      for (int64_t kk = 0; kk < k; ++kk) {
        const float* brow = P.Bw + kk * n + j0;
        for (int64_t ii = 0; ii < ib; ++ii) {
          const float a = P.Aw[(i0 + ii) * k + kk];
          float* ar = acc.data() + ii * JB;
          for (int64_t jj = 0; jj < jb; ++jj) {
            const float prod = a * brow[jj];
            ar[jj] = ar[jj] + prod;
          }
        }
      }
      // epilogue, element by element
      for (int64_t ii = 0; ii < ib; ++ii) {
        const int64_t i = i0 + ii;
        const bool backward = P.epilog == OEP_DRELU_BGRAD || P.epilog == OEP_DRELU_BGRAD_UNFUSED;
        const float bias_i = (P.epilog == OEP_NONE || backward) ? 0.0f : load_elem(P.bias, P.vec_dt, i);
        for (int64_t jj = 0; jj < jb; ++jj) {
          const int64_t j = j0 + jj;
          const float a = acc[(size_t)(ii * JB + jj)];
          const int64_t o = i * n + j;
          switch (P.epilog) {
            case OEP_NONE:
              store_elem(P.D, P.d_dt, o, a);
              if (P.pre_out) P.pre_out[o] = a;
              break;
            case OEP_BIAS: {
              const float pre = a + bias_i;
              store_elem(P.D, P.d_dt, o, pre);
              if (P.pre_out) P.pre_out[o] = pre;
              break;
            }
            case OEP_RELU_BIAS:
            case OEP_RELU_AUX_BIAS: {
              const float pre = a + bias_i;
              store_elem(P.D, P.d_dt, o, relu(pre));
              if (P.pre_out) P.pre_out[o] = pre;
              if (P.epilog == OEP_RELU_AUX_BIAS && pre > 0.0f)
                P.aux[(i / 32) * n + j] |= 1u << (i % 32);
              break;
            }
            case OEP_GELU_BIAS: {
              const float pre = a + bias_i;
              const float y = (float)gelu_tanh((double)pre);
              store_elem(P.D, P.d_dt, o, y);
              if (P.pre_out) P.pre_out[o] = pre;
              break;
            }
            case OEP_DRELU_BGRAD: {
              const uint32_t bit = (P.aux[(i / 32) * n + j] >> (i % 32)) & 1u;
              const float dz = bit ? a : 0.0f;
              store_elem(P.D, P.d_dt, o, dz);
              if (P.pre_out) P.pre_out[o] = dz;
              rowsum[(size_t)ii] += (double)dz;
              rowabs[(size_t)ii] += std::fabs((double)dz);
              break;
            }
            case OEP_RELU_BIAS_UNFUSED: {
              // three separately rounded steps: GEMM -> T1, T1 + bias -> T2, ReLU(T2) -> D
              const float t1 = round_through(P.d_dt, a);
              const float t2 = round_through(P.d_dt, t1 + bias_i);
              store_elem(P.D, P.d_dt, o, relu(t2));
              if (P.pre_out) P.pre_out[o] = t2;
              break;
            }
            case OEP_DRELU_BGRAD_UNFUSED: {
              // GEMM -> T1 (rounded to D's type), then T1 kept where the stored forward
              // activation is positive; the row sums read those stored values
              const float t1 = round_through(P.d_dt, a);
              const float dz = load_elem(P.act, P.d_dt, o) > 0.0f ? t1 : 0.0f;
              store_elem(P.D, P.d_dt, o, dz);
              if (P.pre_out) P.pre_out[o] = dz;
              rowsum[(size_t)ii] += (double)dz;
              rowabs[(size_t)ii] += std::fabs((double)dz);
              break;
            }
          }
        }
      }
    }
    if (P.epilog == OEP_DRELU_BGRAD || P.epilog == OEP_DRELU_BGRAD_UNFUSED) {
      for (int64_t ii = 0; ii < ib; ++ii) {
        store_elem(P.bgrad, P.vec_dt, i0 + ii, (float)rowsum[(size_t)ii]);
        if (P.absum_out) P.absum_out[i0 + ii] = rowabs[(size_t)ii];
      }
    }
  }
}

int default_threads() {
  const char* s = std::getenv("ORACLE_THREADS");
  if (s && std::atoi(s) > 0) return std::atoi(s);
  unsigned hc = std::thread::hardware_concurrency();
  return (int)std::max(1u, std::min(hc, 16u));
}

}  // namespace

extern "C" {

float oracle_f16_to_f32(uint16_t h) { return f16_to_f32(h); }
uint16_t oracle_f32_to_f16(float x) { return f32_to_f16(x); }
float oracle_bf16_to_f32(uint16_t h) { return bf16_to_f32(h); }
uint16_t oracle_f32_to_bf16(float x) { return f32_to_bf16(x); }
double oracle_gelu_tanh(double x) { return gelu_tanh(x); }
int oracle_default_threads(void) { return default_threads(); }

// Bulk conversions used by the pins (n elements).
void oracle_f32_to_f16_n(const float* x, uint16_t* y, int64_t n) { for (int64_t i = 0; i < n; ++i) y[i] = f32_to_f16(x[i]); }
void oracle_f16_to_f32_n(const uint16_t* x, float* y, int64_t n) { for (int64_t i = 0; i < n; ++i) y[i] = f16_to_f32(x[i]); }
void oracle_f32_to_bf16_n(const float* x, uint16_t* y, int64_t n) { for (int64_t i = 0; i < n; ++i) y[i] = f32_to_bf16(x[i]); }
void oracle_bf16_to_f32_n(const uint16_t* x, float* y, int64_t n) { for (int64_t i = 0; i < n; ++i) y[i] = bf16_to_f32(x[i]); }

// Full computation on host memory. A (m,k) (or (k,m) with trans_a), B (k,n) (or
// (n,k) with trans_b), D (m,n), all row-major; bias and bgrad hold m values; aux
// holds ceil(m/32)*n words; act holds the (m,n) forward activation in d_dt, read by
// DRELU_BGRAD_UNFUSED only. Returns 0 on success, -1 on an invalid argument.
// nthreads <= 0 picks min(hardware threads, 16) or $ORACLE_THREADS.
int oracle_gemm_epilog_act_t(int64_t m, int64_t n, int64_t k, int ab_dt, int d_dt, int vec_dt, int epilog,
                             int trans_a, int trans_b, const void* A, const void* B, const void* bias,
                             const void* act, void* D, uint32_t* aux, void* bgrad, float* pre_out,
                             double* absum_out, int nthreads) {
  if (m < 1 || n < 1 || k < 1) return -1;
  if (ab_dt < 0 || ab_dt > 2 || d_dt < 0 || d_dt > 2 || vec_dt < 0 || vec_dt > 2) return -1;
  const bool uses_bias = epilog == OEP_BIAS || epilog == OEP_RELU_BIAS || epilog == OEP_GELU_BIAS ||
                         epilog == OEP_RELU_AUX_BIAS || epilog == OEP_RELU_BIAS_UNFUSED;
  if (!(uses_bias || epilog == OEP_NONE || epilog == OEP_DRELU_BGRAD || epilog == OEP_DRELU_BGRAD_UNFUSED))
    return -1;
  if (!A || !B || !D) return -1;
  if (uses_bias && !bias) return -1;
  if ((epilog == OEP_RELU_AUX_BIAS || epilog == OEP_DRELU_BGRAD) && !aux) return -1;
  if ((epilog == OEP_DRELU_BGRAD || epilog == OEP_DRELU_BGRAD_UNFUSED) && !bgrad) return -1;
  if (epilog == OEP_DRELU_BGRAD_UNFUSED && !act) return -1;

  // O0: widen the operands exactly, into a (m,k) and b (k,n)
  std::vector<float> Aw((size_t)(m * k)), Bw((size_t)(k * n));
  for (int64_t i = 0; i < m; ++i)
    for (int64_t kk = 0; kk < k; ++kk)
      Aw[(size_t)(i * k + kk)] = load_elem(A, ab_dt, trans_a ? kk * m + i : i * k + kk);
  for (int64_t kk = 0; kk < k; ++kk)
    for (int64_t j = 0; j < n; ++j)
      Bw[(size_t)(kk * n + j)] = load_elem(B, ab_dt, trans_b ? j * k + kk : kk * n + j);

  Problem P{m, n, k, ab_dt, d_dt, vec_dt, epilog, Aw.data(), Bw.data(), bias, D, aux, bgrad, act, pre_out, absum_out};
  if (epilog == OEP_RELU_AUX_BIAS && (m % 32) != 0) {
    // pad bits of the last group are zero: clear that group up front
    std::fill(aux + (m / 32) * n, aux + (m / 32 + 1) * n, 0u);
  }

  int nt = nthreads > 0 ? nthreads : default_threads();
  const int64_t groups = (m + 31) / 32;
  nt = (int)std::min<int64_t>(nt, groups);
  std::vector<std::thread> pool;
  for (int t = 0; t < nt; ++t) {
    const int64_t g0 = groups * t / nt, g1 = groups * (t + 1) / nt;
    const int64_t r0 = g0 * 32, r1 = std::min(m, g1 * 32);
    if (r0 >= r1) continue;
    pool.emplace_back([&P, r0, r1] { compute_rows(P, r0, r1); });
  }
  for (auto& th : pool) th.join();
  return 0;
}

// Without the activation argument (every epilogue but DRELU_BGRAD_UNFUSED).
int oracle_gemm_epilog_t(int64_t m, int64_t n, int64_t k, int ab_dt, int d_dt, int vec_dt, int epilog,
                         int trans_a, int trans_b, const void* A, const void* B, const void* bias, void* D,
                         uint32_t* aux, void* bgrad, float* pre_out, double* absum_out, int nthreads) {
  return oracle_gemm_epilog_act_t(m, n, k, ab_dt, d_dt, vec_dt, epilog, trans_a, trans_b, A, B, bias, nullptr, D,
                                  aux, bgrad, pre_out, absum_out, nthreads);
}

// Both operands stored as in the product: A (m,k), B (k,n).
int oracle_gemm_epilog(int64_t m, int64_t n, int64_t k, int ab_dt, int d_dt, int vec_dt, int epilog,
                       const void* A, const void* B, const void* bias, void* D, uint32_t* aux,
                       void* bgrad, float* pre_out, double* absum_out, int nthreads) {
  return oracle_gemm_epilog_t(m, n, k, ab_dt, d_dt, vec_dt, epilog, 0, 0, A, B, bias, D, aux, bgrad, pre_out,
                              absum_out, nthreads);
}

}  // extern "C"
