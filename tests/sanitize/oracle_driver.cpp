// Exercises the CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer (built
// by tests/test_oracle_sanitize.py with g++, host code only): every epilogue, every
// storage type, ragged m (a partial mask word group), transposed operands and several
// thread counts, on small integer-valued inputs; each result is also checked against a
// direct float64 sum, so the run fails on a wrong value as well as on a sanitizer report.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

extern "C" {
int oracle_gemm_epilog_t(int64_t m, int64_t n, int64_t k, int ab_dt, int d_dt, int vec_dt, int epilog, int trans_a,
                         int trans_b, const void* A, const void* B, const void* bias, void* D, uint32_t* aux,
                         void* bgrad, float* pre_out, double* absum_out, int nthreads);
float oracle_f16_to_f32(uint16_t h);
uint16_t oracle_f32_to_f16(float x);
float oracle_bf16_to_f32(uint16_t h);
uint16_t oracle_f32_to_bf16(float x);
}

namespace {

int failures = 0;

void check(bool ok, const char* what, int64_t m, int64_t n, int64_t k, int dt, int ep) {
  if (!ok) {
    std::printf("FAIL %s m=%lld n=%lld k=%lld dt=%d ep=%d\n", what, (long long)m, (long long)n, (long long)k, dt, ep);
    ++failures;
  }
}

// Store an exact small integer in storage type dt.
void put(std::vector<uint8_t>& buf, int dt, int64_t i, float v) {
  if (dt == 0) std::memcpy(buf.data() + 4 * i, &v, 4);
  else {
    const uint16_t h = dt == 1 ? oracle_f32_to_f16(v) : oracle_f32_to_bf16(v);
    std::memcpy(buf.data() + 2 * i, &h, 2);
  }
}
float get(const std::vector<uint8_t>& buf, int dt, int64_t i) {
  if (dt == 0) {
    float v;
    std::memcpy(&v, buf.data() + 4 * i, 4);
    return v;
  }
  uint16_t h;
  std::memcpy(&h, buf.data() + 2 * i, 2);
  return dt == 1 ? oracle_f16_to_f32(h) : oracle_bf16_to_f32(h);
}

void run(int64_t m, int64_t n, int64_t k, int dt, int ta, int tb, int threads) {
  const int es = dt == 0 ? 4 : 2;
  uint32_t s = (uint32_t)(m * 131 + n * 17 + k * 7 + dt);
  auto rnd = [&]() {   // small integers in [-2, 2]
    s = s * 1664525u + 1013904223u;
    return (float)((int)((s >> 16) % 5) - 2);
  };
  std::vector<double> a(m * k), b(k * n), bias(m);
  std::vector<uint8_t> A(m * k * es), B(k * n * es), Bias(m * es), D(m * n * es), G(m * es);
  for (int64_t i = 0; i < m; ++i)
    for (int64_t kk = 0; kk < k; ++kk) {
      a[i * k + kk] = rnd();
      put(A, dt, ta ? kk * m + i : i * k + kk, (float)a[i * k + kk]);
    }
  for (int64_t kk = 0; kk < k; ++kk)
    for (int64_t j = 0; j < n; ++j) {
      b[kk * n + j] = rnd();
      put(B, dt, tb ? j * k + kk : kk * n + j, (float)b[kk * n + j]);
    }
  for (int64_t i = 0; i < m; ++i) {
    bias[i] = rnd() + 0.5;
    put(Bias, dt, i, (float)bias[i]);
  }
  const int64_t groups = (m + 31) / 32;
  std::vector<uint32_t> mask(groups * n, 0xdeadbeefu);
  std::vector<float> pre(m * n);
  std::vector<double> absum(m);
  for (int ep : {0, 1, 2, 3, 5, 100}) {
    const int rc = oracle_gemm_epilog_t(m, n, k, dt, dt, dt, ep, ta, tb, A.data(), B.data(), Bias.data(), D.data(),
                                        mask.data(), nullptr, pre.data(), nullptr, threads);
    check(rc == 0, "rc", m, n, k, dt, ep);
    for (int64_t i = 0; i < m; ++i)
      for (int64_t j = 0; j < n; ++j) {
        double acc = 0;
        for (int64_t kk = 0; kk < k; ++kk) acc += a[i * k + kk] * b[kk * n + j];
        const double p = ep == 0 ? acc : acc + bias[i];
        const double y = (ep == 0 || ep == 5) ? p : ep == 2 ? 0.5 * p * (1 + std::tanh(0.7978845608028654 *
                                                                                    (p + 0.044715 * p * p * p)))
                                                            : (p > 0 ? p : 0);
        const double got = get(D, dt, i * n + j);
        const double tol = ep == 2 ? 0.02 * std::fmax(1.0, std::fabs(y)) : 0.0;
        check(std::fabs(got - y) <= tol, "D", m, n, k, dt, ep);
        if (ep == 3) check((((mask[(i / 32) * n + j] >> (i % 32)) & 1u) != 0) == (p > 0), "mask", m, n, k, dt, ep);
      }
    if (ep == 3)
      for (int64_t i = m; i < groups * 32; ++i)
        for (int64_t j = 0; j < n; ++j) check(((mask[(i / 32) * n + j] >> (i % 32)) & 1u) == 0, "pad", m, n, k, dt, ep);
  }
  // backward on the mask just written
  const int rc = oracle_gemm_epilog_t(m, n, k, dt, dt, dt, 4, ta, tb, A.data(), B.data(), nullptr, D.data(),
                                      mask.data(), G.data(), pre.data(), absum.data(), threads);
  check(rc == 0, "rc bwd", m, n, k, dt, 4);
  for (int64_t i = 0; i < m; ++i) {
    double row = 0;
    for (int64_t j = 0; j < n; ++j) {
      double acc = 0;
      for (int64_t kk = 0; kk < k; ++kk) acc += a[i * k + kk] * b[kk * n + j];
      const double dz = ((mask[(i / 32) * n + j] >> (i % 32)) & 1u) ? acc : 0.0;
      check(get(D, dt, i * n + j) == dz, "dz", m, n, k, dt, 4);
      row += dz;
    }
    check(get(G, dt, i) == row, "bgrad", m, n, k, dt, 4);
  }
}

}  // namespace

int main() {
  for (int dt = 0; dt < 3; ++dt)
    for (int64_t m : {1, 31, 33, 70})
      for (int64_t n : {8, 24})
        for (int64_t k : {1, 8, 13})
          for (int t = 0; t < 4; ++t) run(m, n, k, dt, t & 1, (t >> 1) & 1, 1 + t);
  // argument errors come back as -1 without touching memory
  check(oracle_gemm_epilog_t(0, 8, 8, 1, 1, 1, 1, 0, 0, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                             nullptr, nullptr, 1) == -1, "bad m", 0, 8, 8, 1, 1);
  std::printf("%s (%d failures)\n", failures ? "FAILED" : "ok", failures);
  return failures ? 1 : 0;
}
