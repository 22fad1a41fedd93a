// Host side of the C ABI: offline weight pack (smoothing, SVD split, residual
// quantization), LoRA fold, the smoothing fold of the down projection, and the
// calibration statistic.  Pure C++ (no HIP calls); fp64 internally.
//
// SVD without LAPACK: W_hat = U S V^T is obtained from the Gram matrix of W_hat (the
// smaller of W_hat W_hat^T and W_hat^T W_hat) whose eigenvectors are the singular
// vectors and whose eigenvalues are the squared singular values (ch3chohch3.github.io
// post "从 Smooth Quant 到 SVD Quant", section "SVD 分解": U and V are the eigenvector
// bases of A A^T and A^T A, singular values the square roots of their eigenvalues).
// The symmetric eigenproblem is solved for the top `rank` pairs only: Householder
// reduction to tridiagonal form, bisection on Sturm counts for the eigenvalues,
// inverse iteration (with re-orthogonalization inside clusters) for the eigenvectors,
// then the Householder back-transformation.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <thread>
#include <vector>

#include "../../include/svdq.h"
#include "internal.hpp"

namespace svdq {
namespace {

int num_threads() {
  const char* env = std::getenv("SVDQ_NUM_THREADS");
  if (!env || !*env) env = std::getenv("OMP_NUM_THREADS");
  int n = env ? std::atoi(env) : 0;
  if (n <= 0) n = (int)std::thread::hardware_concurrency();
  return std::max(1, std::min(n, 64));
}

// Run f(i) for i in [0, n) on a fresh set of threads (coarse-grained phases only).
template <class F>
void parallel_for(int64_t n, F&& f) {
  const int nt = (int)std::min<int64_t>(num_threads(), std::max<int64_t>(n, 1));
  if (nt <= 1) {
    for (int64_t i = 0; i < n; ++i) f(i);
    return;
  }
  std::atomic<int64_t> next{0};
  std::vector<std::thread> th;
  for (int t = 0; t < nt; ++t)
    th.emplace_back([&] {
      for (int64_t i; (i = next.fetch_add(1)) < n;) f(i);
    });
  for (auto& x : th) x.join();
}

// Sense-reversing spin barrier for the SPMD tridiagonal reduction.
class SpinBarrier {
 public:
  explicit SpinBarrier(int n) : n_(n), count_(n), sense_(0) {}
  void wait() {
    const int s = sense_.load(std::memory_order_relaxed);
    if (count_.fetch_sub(1, std::memory_order_acq_rel) == 1) {
      count_.store(n_, std::memory_order_relaxed);
      sense_.store(s ^ 1, std::memory_order_release);
    } else {
      int spins = 0;
      while (sense_.load(std::memory_order_acquire) == s)
        if (++spins > 4096) std::this_thread::yield();
    }
  }

 private:
  const int n_;
  std::atomic<int> count_;
  std::atomic<int> sense_;
};

// ---------------------------------------------------------------- number formats
inline double bf16_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return (double)f;
}
inline float bf16_to_float(uint16_t b) { return (float)bf16_to_double(b); }

// fp64 -> bf16, round to nearest even in a single step.
uint16_t double_to_bf16(double x) {
  if (x == 0.0 || std::isnan(x)) return std::signbit(x) ? 0x8000 : (std::isnan(x) ? 0x7FC0 : 0);
  int e;
  std::frexp(x, &e);  // x = f 2^e, f in [0.5, 1)
  const int be = std::max(e - 1, -126);
  const double q = std::ldexp(1.0, be - 7);
  const double r = std::nearbyint(x / q) * q;
  float f = std::fabs(r) >= 0x1p128 ? std::copysign(std::numeric_limits<float>::infinity(), r) : (float)r;
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

// fp32 -> fp16 bits, round to nearest even, overflow saturating to 65504.
uint16_t float_to_f16_sat(float f) {
  const double x = f;
  const uint16_t sign = std::signbit(x) ? 0x8000 : 0;
  const double ax = std::fabs(x);
  if (ax == 0.0) return sign;
  int e;
  std::frexp(ax, &e);
  const int be = std::max(e - 1, -14);
  const double q = std::ldexp(1.0, be - 10);
  double r = std::nearbyint(ax / q) * q;
  if (r > 65504.0) r = 65504.0;
  if (r < 0x1p-14) return (uint16_t)(sign | (uint16_t)std::lrint(r / 0x1p-24));
  int re;
  std::frexp(r, &re);
  const int ex = re - 1;  // r in [2^ex, 2^(ex+1))
  const int mant = (int)std::lrint((r / std::ldexp(1.0, ex) - 1.0) * 1024.0);
  return (uint16_t)(sign | ((ex + 15) << 10) | mant);
}

double f16_to_double(uint16_t b) {
  const int s = b >> 15, e = (b >> 10) & 0x1F, m = b & 0x3FF;
  double v = (e == 0) ? std::ldexp((double)m, -24) : std::ldexp(1.0 + m / 1024.0, e - 15);
  return s ? -v : v;
}

// ------------------------------------------------------------------ quantizers
// INT4 group: s = fp16(fp32(max|v| / 7)), q = round-half-even(v / s) exactly (the fp64
// quotient of an fp32 value by an fp16 value cannot cross a half-integer), clamped
// to [-7, 7]; nibble = sign << 3 | |q|.
void quant_int4_group(const float* v, int G, uint8_t* nib, uint16_t* sbits) {
  float a = 0.f;
  for (int i = 0; i < G; ++i) a = std::max(a, std::fabs(v[i]));
  const float s32 = a / 7.0f;
  const uint16_t sb = float_to_f16_sat(s32);
  const double s = f16_to_double(sb);
  for (int i = 0; i < G; ++i) {
    int q = 0;
    if (s != 0.0) {
      double t = std::nearbyint((double)v[i] / s);
      t = std::min(7.0, std::max(-7.0, t));
      q = (int)t;
    }
    nib[i] = (uint8_t)((q < 0 ? 8 : 0) | std::abs(q));
  }
  *sbits = sb;
}

// FP4 group: e = smallest exponent with 6 * 2^e >= max|v| (0 for an all-zero group),
// clamped to [-127, 127]; code = sign << 3 | E2M1 index of round-half-even(v * 2^-e).
void quant_fp4_group(const float* v, int G, uint8_t* nib, uint8_t* e8) {
  float a = 0.f;
  for (int i = 0; i < G; ++i) a = std::max(a, std::fabs(v[i]));
  int e = 0;
  if (a != 0.f) {
    int E;
    const double f = std::frexp((double)a, &E);  // a = f 2^E, f in [0.5, 1)
    const double m = 2.0 * f;
    const int Eb = E - 1;
    e = (m <= 1.5) ? Eb - 2 : Eb - 1;
    e = std::max(-127, std::min(127, e));
  }
  for (int i = 0; i < G; ++i) {
    const double u = std::fabs(std::ldexp((double)v[i], -e));
    int idx;
    if (u <= 0.25) idx = 0;
    else if (u < 0.75) idx = 1;
    else if (u <= 1.25) idx = 2;
    else if (u < 1.75) idx = 3;
    else if (u <= 2.5) idx = 4;
    else if (u < 3.5) idx = 5;
    else if (u <= 5.0) idx = 6;
    else idx = 7;
    nib[i] = (uint8_t)((std::signbit(v[i]) ? 8 : 0) | idx);
  }
  *e8 = (uint8_t)(e + 127);
}

// Non-negative x -> the nearest FP8 E4M3 value (bias 7, 3 mantissa bits, subnormals
// m 2^-9), ties to the even mantissa, saturating at 448; returns the code byte.
uint8_t e4m3_rne_sat(double x) {
  if (!(x > 0.0)) return 0;
  int e;
  std::frexp(x, &e);  // x = f 2^e, f in [0.5, 1): binary exponent e - 1
  const int be = std::max(e - 1, -6);
  double r = std::nearbyint(std::ldexp(x, 3 - be));  // quanta of 2^(be - 3)
  double v = std::ldexp(r, be - 3);
  if (v >= 448.0) return 0x7E;
  if (v < 0x1p-6) return (uint8_t)std::lrint(std::ldexp(v, 9));  // subnormal (or 0)
  int re;
  std::frexp(v, &re);
  const int ex = re - 1;
  const int mant = (int)std::lrint((std::ldexp(v, -ex) - 1.0) * 8.0);
  return (uint8_t)(((ex + 7) << 3) | mant);
}

double e4m3_to_double(uint8_t b) {
  const int E = (b >> 3) & 15, m = b & 7;
  return E == 0 ? std::ldexp((double)m, -9) : std::ldexp(1.0 + m / 8.0, E - 7);
}

// E2M1 magnitude index of u >= 0: round half to even on {0, .5, 1, 1.5, 2, 3, 4, 6},
// saturating at 6.
int e2m1_index(double u) {
  if (u <= 0.25) return 0;
  if (u < 0.75) return 1;
  if (u <= 1.25) return 2;
  if (u < 1.75) return 3;
  if (u <= 2.5) return 4;
  if (u < 3.5) return 5;
  if (u <= 5.0) return 6;
  return 7;
}

// NVFP4 level-2 scale fp32(amax / 2688) (1 for amax = 0).
float nv_tensor_scale(float amax) { return amax == 0.f ? 1.f : amax / 2688.0f; }

// NVFP4 group of 16 under the tensor scale S (r6 = fp32(1 / fp32(6 S))): s =
// E4M3(fp32(a r6)), sigma = fp32(s S), code = E2M1 of fp32(v * fp32(1 / sigma)).
void quant_nv_group(const float* v, float S, float r6, uint8_t* nib, uint8_t* e4) {
  float a = 0.f;
  for (int i = 0; i < 16; ++i) a = std::max(a, std::fabs(v[i]));
  const float t = a * r6;
  const uint8_t sb = e4m3_rne_sat((double)t);
  const float sigma = (float)e4m3_to_double(sb) * S;
  const float rcp = sigma > 0.f ? 1.0f / sigma : 0.f;
  for (int i = 0; i < 16; ++i) {
    const float q = v[i] * rcp;
    nib[i] = (uint8_t)((std::signbit(v[i]) ? 8 : 0) | e2m1_index(std::fabs((double)q)));
  }
  *e4 = sb;
}

// Quantize R [K][N] (fp32, row-major) per column along K; write qW [N][K/2], sW [K/G][N]
// (NVFP4: then the fp32 tensor scale of R and the activations' S_X).
void quantize_residual(int64_t K, int64_t N, const float* R, int fmt, uint8_t* qW, void* sW, float S_X = 1.f) {
  const int G = group_of(fmt);
  const int64_t ng = K / G;
  float S = 1.f, r6 = 0.f;
  if (fmt == SVDQ_NVFP4_G16) {
    float amax = 0.f;
    for (int64_t i = 0; i < K * N; ++i) amax = std::max(amax, std::fabs(R[i]));
    S = nv_tensor_scale(amax);
    r6 = 1.0f / (6.0f * S);
    uint8_t* tail = static_cast<uint8_t*>(sW) + ng * N;
    std::memcpy(tail, &S, 4);
    std::memcpy(tail + 4, &S_X, 4);
  }
  parallel_for((N + 63) / 64, [&](int64_t blk) {
    std::vector<float> col(K);
    std::vector<uint8_t> nib(K);
    for (int64_t n = blk * 64; n < std::min(N, blk * 64 + 64); ++n) {
      for (int64_t k = 0; k < K; ++k) col[k] = R[k * N + n];
      for (int64_t g = 0; g < ng; ++g) {
        if (fmt == SVDQ_INT4_G64) {
          uint16_t sb;
          quant_int4_group(&col[g * G], G, &nib[g * G], &sb);
          static_cast<uint16_t*>(sW)[g * N + n] = sb;
        } else if (fmt == SVDQ_NVFP4_G16) {
          uint8_t e4;
          quant_nv_group(&col[g * G], S, r6, &nib[g * G], &e4);
          static_cast<uint8_t*>(sW)[g * N + n] = e4;
        } else {
          uint8_t e8;
          quant_fp4_group(&col[g * G], G, &nib[g * G], &e8);
          static_cast<uint8_t*>(sW)[g * N + n] = e8;
        }
      }
      uint8_t* q = qW + n * (K / 2);
      for (int64_t j = 0; j < K / 2; ++j) q[j] = (uint8_t)(nib[2 * j] | (nib[2 * j + 1] << 4));
    }
  });
}

// ------------------------------------------------------------- symmetric eigen
// G = A A^T for A [n][L] (row-major, rows are the vectors): lower triangle + mirror.
void gram(const double* A, int64_t n, int64_t L, double* G) {
  const int64_t B = 64;
  const int64_t nb = (n + B - 1) / B;
  std::vector<std::pair<int64_t, int64_t>> tiles;
  for (int64_t bi = 0; bi < nb; ++bi)
    for (int64_t bj = 0; bj <= bi; ++bj) tiles.emplace_back(bi, bj);
  parallel_for((int64_t)tiles.size(), [&](int64_t t) {
    const int64_t i0 = tiles[t].first * B, j0 = tiles[t].second * B;
    const int64_t i1 = std::min(n, i0 + B), j1 = std::min(n, j0 + B);
    double acc[B][B];
    for (int64_t i = 0; i < B; ++i)
      for (int64_t j = 0; j < B; ++j) acc[i][j] = 0.0;
    const int64_t LC = 256;
    for (int64_t l0 = 0; l0 < L; l0 += LC) {
      const int64_t l1 = std::min(L, l0 + LC);
      for (int64_t i = i0; i < i1; i += 4) {
        for (int64_t j = j0; j < j1; j += 4) {
          double s[4][4] = {};
          const int64_t ni = std::min<int64_t>(4, i1 - i), nj = std::min<int64_t>(4, j1 - j);
          if (ni == 4 && nj == 4) {
            const double *a0 = A + i * L, *a1 = a0 + L, *a2 = a1 + L, *a3 = a2 + L;
            const double *b0 = A + j * L, *b1 = b0 + L, *b2 = b1 + L, *b3 = b2 + L;
            for (int64_t l = l0; l < l1; ++l) {
              const double x0 = a0[l], x1 = a1[l], x2 = a2[l], x3 = a3[l];
              const double y0 = b0[l], y1 = b1[l], y2 = b2[l], y3 = b3[l];
              s[0][0] += x0 * y0; s[0][1] += x0 * y1; s[0][2] += x0 * y2; s[0][3] += x0 * y3;
              s[1][0] += x1 * y0; s[1][1] += x1 * y1; s[1][2] += x1 * y2; s[1][3] += x1 * y3;
              s[2][0] += x2 * y0; s[2][1] += x2 * y1; s[2][2] += x2 * y2; s[2][3] += x2 * y3;
              s[3][0] += x3 * y0; s[3][1] += x3 * y1; s[3][2] += x3 * y2; s[3][3] += x3 * y3;
            }
          } else {
            for (int64_t a = 0; a < ni; ++a)
              for (int64_t b = 0; b < nj; ++b) {
                const double* x = A + (i + a) * L;
                const double* y = A + (j + b) * L;
                double t2 = 0.0;
                for (int64_t l = l0; l < l1; ++l) t2 += x[l] * y[l];
                s[a][b] = t2;
              }
          }
          for (int64_t a = 0; a < ni; ++a)
            for (int64_t b = 0; b < nj; ++b) acc[i - i0 + a][j - j0 + b] += s[a][b];
        }
      }
    }
    for (int64_t i = i0; i < i1; ++i)
      for (int64_t j = j0; j < j1; ++j) {
        G[i * n + j] = acc[i - i0][j - j0];
        G[j * n + i] = acc[i - i0][j - j0];
      }
  });
}

// Householder reduction of the symmetric matrix A [n][n] (full storage, overwritten)
// to tridiagonal form: d [n] diagonal, e [n-1] off-diagonal.  Reflector k is
// H_k = I - beta[k] v v^T acting on indices k+1.., with v stored in A[k+1..][k].
void tridiagonalize(double* A, int64_t n, double* d, double* e, double* beta) {
  const int nt = (int)std::max<int64_t>(1, std::min<int64_t>(num_threads(), n / 64));
  std::vector<double> v(n), p(n), w(n);
  double bshared = 0.0;
  SpinBarrier bar(nt);
  auto worker = [&](int tid) {
    for (int64_t k = 0; k + 2 < n; ++k) {
      const int64_t s = k + 1;  // trailing block starts here
      if (tid == 0) {
        double nrm2 = 0.0;
        for (int64_t i = s; i < n; ++i) nrm2 += A[i * n + k] * A[i * n + k];
        const double x0 = A[s * n + k];
        const double nrm = std::sqrt(nrm2);
        d[k] = A[k * n + k];
        if (nrm == 0.0) {
          bshared = 0.0;
          e[k] = 0.0;
          for (int64_t i = s; i < n; ++i) v[i] = 0.0;
        } else {
          const double alpha = x0 >= 0 ? -nrm : nrm;
          for (int64_t i = s; i < n; ++i) v[i] = A[i * n + k];
          v[s] = x0 - alpha;
          const double vtv = nrm2 - x0 * x0 + v[s] * v[s];
          bshared = vtv > 0 ? 2.0 / vtv : 0.0;
          e[k] = alpha;
        }
        beta[k] = bshared;
        for (int64_t i = s; i < n; ++i) A[i * n + k] = v[i];
      }
      bar.wait();
      const double b = bshared;
      if (b != 0.0) {
        for (int64_t i = s + tid; i < n; i += nt) {
          const double* row = A + i * n;
          double acc = 0.0;
          for (int64_t j = s; j < n; ++j) acc += row[j] * v[j];
          p[i] = b * acc;
        }
      }
      bar.wait();
      if (b != 0.0) {
        if (tid == 0) {
          double pv = 0.0;
          for (int64_t i = s; i < n; ++i) pv += p[i] * v[i];
          const double Kc = 0.5 * b * pv;
          for (int64_t i = s; i < n; ++i) w[i] = p[i] - Kc * v[i];
        }
        bar.wait();
        for (int64_t i = s + tid; i < n; i += nt) {
          double* row = A + i * n;
          const double vi = v[i], wi = w[i];
          for (int64_t j = s; j < n; ++j) row[j] -= vi * w[j] + wi * v[j];
        }
      }
      bar.wait();
    }
  };
  std::vector<std::thread> th;
  for (int t = 1; t < nt; ++t) th.emplace_back(worker, t);
  worker(0);
  for (auto& x : th) x.join();
  if (n >= 2) {
    d[n - 2] = A[(n - 2) * n + (n - 2)];
    d[n - 1] = A[(n - 1) * n + (n - 1)];
    e[n - 2] = A[(n - 1) * n + (n - 2)];
    beta[n - 2] = 0.0;
    if (n >= 2) beta[n - 1] = 0.0;
  } else if (n == 1) {
    d[0] = A[0];
    beta[0] = 0.0;
  }
}

// Number of eigenvalues of the tridiagonal (d, e) strictly below x (Sturm count).
int64_t sturm_count(const double* d, const double* e2, int64_t n, double x, double pivmin) {
  int64_t c = 0;
  double q = d[0] - x;
  if (std::fabs(q) < pivmin) q = -pivmin;
  if (q < 0) ++c;
  for (int64_t i = 1; i < n; ++i) {
    q = d[i] - x - e2[i - 1] / q;
    if (std::fabs(q) < pivmin) q = -pivmin;
    if (q < 0) ++c;
  }
  return c;
}

// Eigenvector of tridiagonal (d, e) for eigenvalue lam by inverse iteration,
// re-orthogonalized against `prev` vectors (same cluster).
void inverse_iteration(const double* d, const double* e, int64_t n, double lam, double tnorm,
                       const std::vector<const double*>& prev, double* x) {
  std::vector<double> D(n), U1(n), U2(n), Lm(n), y(n);
  std::vector<char> piv(n);
  const double eps = std::numeric_limits<double>::epsilon();
  const double pert = std::max(eps * tnorm, std::numeric_limits<double>::min());
  for (int64_t i = 0; i < n; ++i) {
    D[i] = d[i] - lam;
    U1[i] = i + 1 < n ? e[i] : 0.0;
    U2[i] = 0.0;
  }
  for (int64_t i = 0; i + 1 < n; ++i) {
    const double c = e[i];
    if (std::fabs(D[i]) >= std::fabs(c)) {
      piv[i] = 0;
      if (D[i] == 0.0) D[i] = pert;
      const double mlt = c / D[i];
      Lm[i] = mlt;
      D[i + 1] -= mlt * U1[i];
    } else {
      piv[i] = 1;
      const double mlt = D[i] / c;
      Lm[i] = mlt;
      const double dn = D[i + 1];
      const double un = (i + 2 < n) ? U1[i + 1] : 0.0;
      D[i] = c;
      D[i + 1] = U1[i] - mlt * dn;
      if (i + 2 < n) U1[i + 1] = -mlt * un;
      U1[i] = dn;
      U2[i] = un;
    }
  }
  if (D[n - 1] == 0.0) D[n - 1] = pert;
  // deterministic start vector
  for (int64_t i = 0; i < n; ++i) x[i] = 1.0 + 0.5 * std::sin(0.7 * (double)i + 0.3 * lam / (tnorm + 1e-300));
  for (int it = 0; it < 4; ++it) {
    for (int64_t i = 0; i < n; ++i) y[i] = x[i];
    for (int64_t i = 0; i + 1 < n; ++i) {
      if (piv[i]) std::swap(y[i], y[i + 1]);
      y[i + 1] -= Lm[i] * y[i];
    }
    for (int64_t i = n - 1; i >= 0; --i) {
      double t = y[i];
      if (i + 1 < n) t -= U1[i] * y[i + 1];
      if (i + 2 < n) t -= U2[i] * y[i + 2];
      y[i] = t / D[i];
    }
    for (const double* p : prev) {
      double dot = 0.0;
      for (int64_t i = 0; i < n; ++i) dot += p[i] * y[i];
      for (int64_t i = 0; i < n; ++i) y[i] -= dot * p[i];
    }
    double nrm = 0.0;
    for (int64_t i = 0; i < n; ++i) nrm += y[i] * y[i];
    nrm = std::sqrt(nrm);
    if (nrm == 0.0 || !std::isfinite(nrm)) {
      for (int64_t i = 0; i < n; ++i) y[i] = (i == 0);
      nrm = 1.0;
    }
    for (int64_t i = 0; i < n; ++i) x[i] = y[i] / nrm;
  }
}

// Top-r eigenpairs (descending) of symmetric G [n][n] (destroyed).  vals [r], vecs [r][n].
void top_eigen(double* G, int64_t n, int64_t r, double* vals, double* vecs) {
  std::vector<double> d(n), e(std::max<int64_t>(n - 1, 1)), beta(n);
  tridiagonalize(G, n, d.data(), e.data(), beta.data());
  std::vector<double> e2(std::max<int64_t>(n - 1, 1));
  double lo = d[0], hi = d[0], tnorm = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    const double r1 = (i > 0 ? std::fabs(e[i - 1]) : 0.0) + (i + 1 < n ? std::fabs(e[i]) : 0.0);
    lo = std::min(lo, d[i] - r1);
    hi = std::max(hi, d[i] + r1);
    tnorm = std::max(tnorm, std::fabs(d[i]) + r1);
  }
  for (int64_t i = 0; i + 1 < n; ++i) e2[i] = e[i] * e[i];
  const double eps = std::numeric_limits<double>::epsilon();
  const double pivmin = std::max(std::numeric_limits<double>::min(), eps * eps * tnorm * tnorm) + 1e-300;
  lo -= 2 * eps * tnorm + pivmin;
  hi += 2 * eps * tnorm + pivmin;
  parallel_for(r, [&](int64_t t) {
    const int64_t j = n - 1 - t;  // ascending index
    double a = lo, b = hi;
    for (int it = 0; it < 200; ++it) {
      const double mid = 0.5 * (a + b);
      if (mid <= a || mid >= b) break;
      if (sturm_count(d.data(), e2.data(), n, mid, pivmin) > j) b = mid;
      else a = mid;
      if (b - a <= 2 * eps * std::max(std::fabs(a), std::fabs(b)) + pivmin) break;
    }
    vals[t] = 0.5 * (a + b);
  });
  // eigenvectors of T, sequential over clusters
  std::vector<double> X((size_t)r * n);
  int64_t cstart = 0;
  for (int64_t t = 0; t < r; ++t) {
    if (t > 0 && std::fabs(vals[t] - vals[t - 1]) > 1e-3 * tnorm) cstart = t;
    std::vector<const double*> prev;
    for (int64_t u = cstart; u < t; ++u) prev.push_back(&X[(size_t)u * n]);
    inverse_iteration(d.data(), e.data(), n, vals[t], tnorm, prev, &X[(size_t)t * n]);
  }
  // back-transformation z = H_0 H_1 ... H_{n-3} x
  parallel_for(r, [&](int64_t t) {
    double* z = &X[(size_t)t * n];
    for (int64_t k = n - 3; k >= 0; --k) {
      const double b = beta[k];
      if (b == 0.0) continue;
      double s = 0.0;
      for (int64_t i = k + 1; i < n; ++i) s += G[i * n + k] * z[i];
      s *= b;
      for (int64_t i = k + 1; i < n; ++i) z[i] -= s * G[i * n + k];
    }
    std::memcpy(vecs + (size_t)t * n, z, sizeof(double) * n);
  });
}

}  // namespace
}  // namespace svdq

using namespace svdq;

extern "C" {

svdq_status svdq_act_absmax(int64_t M, int64_t K, const uint16_t* X, int64_t ldx, float* out) {
  if (!X || !out) return fail(SVDQ_EINVAL, "X and out must be non-NULL");
  if (M < 1 || K < 1 || ldx < K) return fail(SVDQ_EINVAL, "need M >= 1, K >= 1, ldx >= K");
  for (int64_t k = 0; k < K; ++k) out[k] = 0.f;
  for (int64_t m = 0; m < M; ++m)
    for (int64_t k = 0; k < K; ++k) out[k] = std::max(out[k], std::fabs(bf16_to_float(X[m * ldx + k])));
  return ok();
}

svdq_status svdq_weight_sizes(int64_t K, int64_t N, int32_t fmt, size_t* qW_bytes, size_t* sW_bytes) {
  svdq_status st = check_dims(K, N, fmt);
  if (st != SVDQ_OK) return st;
  if (!qW_bytes || !sW_bytes) return fail(SVDQ_EINVAL, "output pointers must be non-NULL");
  *qW_bytes = (size_t)N * (size_t)(K / 2);
  *sW_bytes = (size_t)(K / group_of(fmt)) * (size_t)N * (fmt == SVDQ_INT4_G64 ? 2 : 1) +
              (fmt == SVDQ_NVFP4_G16 ? 8 : 0);
  return ok();
}

svdq_status svdq_quantize_weights(int64_t K, int64_t N, const float* R, int32_t fmt, uint8_t* qW_out,
                                  void* sW_out) {
  svdq_status st = check_dims(K, N, fmt);
  if (st != SVDQ_OK) return st;
  if (!R || !qW_out || !sW_out) return fail(SVDQ_EINVAL, "R, qW_out and sW_out must be non-NULL");
  for (int64_t i = 0; i < K * N; ++i)
    if (!std::isfinite(R[i])) return fail(SVDQ_ENUMERIC, "R has a non-finite value at %lld", (long long)i);
  quantize_residual(K, N, R, fmt, qW_out, sW_out);
  return ok();
}

}  // extern "C"

namespace svdq {
namespace {

// Rank-r split of a target T [K][N] (fp64) from the Gram matrix of its smaller side:
// L1 = U_r Sigma_r, L2 = V_r^T, both rounded to bf16 (bits into L1t_bits [rank][K],
// L2_bits [rank][N]; values into L1 [K][rank], L2 [rank][N]).
void split_rank(const double* T, int64_t K, int64_t N, int32_t rank, std::vector<double>& L1,
                std::vector<double>& L2, uint16_t* L1t_bits, uint16_t* L2_bits) {
  const bool left = K <= N;
  const int64_t n = left ? K : N, L = left ? N : K;
  std::vector<double> At;
  const double* A = T;
  if (!left) {
    At.resize((size_t)N * K);
    parallel_for(N, [&](int64_t c) {
      for (int64_t k = 0; k < K; ++k) At[c * K + k] = T[k * N + c];
    });
    A = At.data();
  }
  std::vector<double> G((size_t)n * n);
  gram(A, n, L, G.data());
  std::vector<double> vals(rank), vecs((size_t)rank * n);
  top_eigen(G.data(), n, rank, vals.data(), vecs.data());
  const double smax = std::sqrt(std::max(vals[0], 0.0));
  parallel_for(rank, [&](int64_t t) {
    const double sig = std::sqrt(std::max(vals[t], 0.0));
    const double* q = &vecs[(size_t)t * n];
    const bool keep = sig > 1e-300 && sig > 1e-15 * smax;
    if (left) {  // q = u_t;  L1[:,t] = sig u_t;  L2[t,:] = T^T u_t / sig
      for (int64_t k = 0; k < K; ++k) L1[k * rank + t] = keep ? sig * q[k] : 0.0;
      for (int64_t c = 0; c < N; ++c) {
        double acc = 0.0;
        if (keep)
          for (int64_t k = 0; k < K; ++k) acc += T[k * N + c] * q[k];
        L2[t * N + c] = keep ? acc / sig : 0.0;
      }
    } else {  // q = v_t;  L2[t,:] = v_t;  L1[:,t] = T v_t
      for (int64_t c = 0; c < N; ++c) L2[t * N + c] = keep ? q[c] : 0.0;
      for (int64_t k = 0; k < K; ++k) {
        double acc = 0.0;
        if (keep)
          for (int64_t c = 0; c < N; ++c) acc += T[k * N + c] * q[c];
        L1[k * rank + t] = acc;
      }
    }
  });
  for (int64_t k = 0; k < K; ++k)
    for (int64_t t = 0; t < rank; ++t) {
      const uint16_t b = double_to_bf16(L1[k * rank + t]);
      L1t_bits[t * K + k] = b;
      L1[k * rank + t] = bf16_to_double(b);
    }
  for (int64_t t = 0; t < rank; ++t)
    for (int64_t c = 0; c < N; ++c) {
      const uint16_t b = double_to_bf16(L2[t * N + c]);
      L2_bits[t * N + c] = b;
      L2[t * N + c] = bf16_to_double(b);
    }
}

// deq(Q(R)) [K][N] from codes qW [N][K/2] and scales sW [K/G][N].
void dequantize_residual(int64_t K, int64_t N, int fmt, const uint8_t* qW, const void* sW, double* D) {
  static const double kE2M1[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
  const int G = group_of(fmt);
  float S = 1.f;
  if (fmt == SVDQ_NVFP4_G16) std::memcpy(&S, static_cast<const uint8_t*>(sW) + (K / G) * N, 4);
  parallel_for(N, [&](int64_t n) {
    for (int64_t k = 0; k < K; ++k) {
      const uint8_t byte = qW[n * (K / 2) + k / 2];
      const int nib = (k & 1) ? byte >> 4 : byte & 15;
      const int64_t g = k / G;
      double v;
      if (fmt == SVDQ_INT4_G64) v = (double)(nib & 7) * f16_to_double(static_cast<const uint16_t*>(sW)[g * N + n]);
      else if (fmt == SVDQ_NVFP4_G16)
        v = kE2M1[nib & 7] * e4m3_to_double(static_cast<const uint8_t*>(sW)[g * N + n]) * (double)S;
      else v = std::ldexp(kE2M1[nib & 7], (int)static_cast<const uint8_t*>(sW)[g * N + n] - 127);
      D[k * N + n] = (nib & 8) ? -v : v;
    }
  });
}

// The pack with `iters` refinement iterates after the plain split (iters = 0: the plain
// split alone); each iterate's E into err_out[t] when given.
svdq_status pack_impl(int64_t K, int64_t N, const uint16_t* W, const float* act_absmax, float alpha, int32_t rank,
                      int32_t fmt, int32_t iters, float* s_out, float* inv_s_out, uint16_t* L1t_out, uint16_t* L2_out,
                      uint8_t* qW_out, void* sW_out, float* R_out, double* err_out) {
  svdq_status st = check_dims(K, N, fmt);
  if (st != SVDQ_OK) return st;
  if (!W || !s_out || !inv_s_out || !qW_out || !sW_out) return fail(SVDQ_EINVAL, "required pointer is NULL");
  if (!(alpha >= 0.f && alpha <= 1.f)) return fail(SVDQ_EINVAL, "alpha must be in [0, 1]");
  if (rank < 0 || rank > SVDQ_MAX_RANK || rank > std::min(K, N))
    return fail(SVDQ_EINVAL, "rank must be in [0, min(K, N, %d)]", SVDQ_MAX_RANK);
  if (rank > 0 && (!L1t_out || !L2_out)) return fail(SVDQ_EINVAL, "L1t_out and L2_out required when rank > 0");
  if (iters < 0 || iters > 64) return fail(SVDQ_EINVAL, "iters must be in [0, 64]");
  for (int64_t i = 0; i < K * N; ++i)
    if (!std::isfinite(bf16_to_double(W[i]))) return fail(SVDQ_ENUMERIC, "W has a non-finite value at %lld", (long long)i);
  if (act_absmax)
    for (int64_t k = 0; k < K; ++k)
      if (!std::isfinite(act_absmax[k])) return fail(SVDQ_ENUMERIC, "act_absmax has a non-finite value");

  // smoothing factor and W_hat = diag(fp32(s)) W
  std::vector<double> What((size_t)K * N);
  for (int64_t k = 0; k < K; ++k) {
    float s32 = 1.f;
    if (act_absmax) {
      double w = 0.0;
      for (int64_t n = 0; n < N; ++n) w = std::max(w, std::fabs(bf16_to_double(W[k * N + n])));
      const double a = std::max((double)act_absmax[k], 1e-5);
      w = std::max(w, 1e-5);
      const double al = (double)alpha;
      s32 = (float)(std::pow(a, al) / std::pow(w, 1.0 - al));
    }
    s_out[k] = s32;
    inv_s_out[k] = 1.0f / s32;
  }
  parallel_for(K, [&](int64_t k) {
    const double s = (double)s_out[k];
    for (int64_t n = 0; n < N; ++n) What[k * N + n] = s * bf16_to_double(W[k * N + n]);
  });

  const int G = group_of(fmt);
  const size_t nq = (size_t)N * (K / 2),
               ns = (size_t)(K / G) * N * (fmt == SVDQ_INT4_G64 ? 2 : 1) + (fmt == SVDQ_NVFP4_G16 ? 8 : 0);
  // NVFP4: the activations' tensor scale from the smoothed calibration statistic
  float S_X = 1.f;
  if (fmt == SVDQ_NVFP4_G16 && act_absmax) {
    float amax = 0.f;
    for (int64_t k = 0; k < K; ++k) amax = std::max(amax, act_absmax[k] * inv_s_out[k]);
    S_X = nv_tensor_scale(amax);
  }
  std::vector<double> L1((size_t)K * std::max(rank, 1)), L2((size_t)std::max(rank, 1) * N);
  std::vector<uint16_t> b1((size_t)std::max(rank, 1) * K), b2((size_t)std::max(rank, 1) * N);
  std::vector<double> Rd((size_t)K * N), D, T;
  std::vector<float> R32((size_t)K * N);
  std::vector<uint8_t> q(nq), sc(ns);
  if (iters > 0) {
    D.resize((size_t)K * N);
    T.resize((size_t)K * N);
  }
  double best = 0.0;
  for (int32_t it = 0; it <= iters; ++it) {
    // iterate 0 splits W_hat; iterate t >= 1 splits W_hat - deq(Q(R_{t-1}))
    const double* target = it == 0 ? What.data() : T.data();
    if (rank > 0) split_rank(target, K, N, rank, L1, L2, b1.data(), b2.data());
    // R = W_hat - L1b L2b with the rounded factors
    parallel_for(K, [&](int64_t k) {
      for (int64_t c = 0; c < N; ++c) {
        double acc = 0.0;
        for (int64_t t = 0; t < rank; ++t) acc += L1[k * rank + t] * L2[t * N + c];
        Rd[k * N + c] = What[k * N + c] - acc;
      }
    });
    for (size_t i = 0; i < R32.size(); ++i) R32[i] = (float)Rd[i];
    quantize_residual(K, N, R32.data(), fmt, q.data(), sc.data(), S_X);
    double err = 0.0;
    if (iters > 0 || err_out) {
      if (D.empty()) D.resize((size_t)K * N);
      dequantize_residual(K, N, fmt, q.data(), sc.data(), D.data());
      std::vector<double> row(K);
      parallel_for(K, [&](int64_t k) {
        double a = 0.0;
        for (int64_t c = 0; c < N; ++c) {
          const double d = Rd[k * N + c] - D[k * N + c];
          a += d * d;
        }
        row[k] = a;
      });
      for (int64_t k = 0; k < K; ++k) err += row[k];  // fixed order
      err = std::sqrt(err);
      if (err_out) err_out[it] = err;
    }
    if (it == 0 || err < best) {  // keep the first iterate with the smallest error
      best = err;
      if (rank > 0) {
        std::memcpy(L1t_out, b1.data(), sizeof(uint16_t) * (size_t)rank * K);
        std::memcpy(L2_out, b2.data(), sizeof(uint16_t) * (size_t)rank * N);
      }
      std::memcpy(qW_out, q.data(), nq);
      std::memcpy(sW_out, sc.data(), ns);
      if (R_out) std::memcpy(R_out, R32.data(), sizeof(float) * R32.size());
    }
    if (it < iters)
      parallel_for(K, [&](int64_t k) {
        for (int64_t c = 0; c < N; ++c) T[k * N + c] = What[k * N + c] - D[k * N + c];
      });
  }
  return ok();
}

}  // namespace
}  // namespace svdq

extern "C" {

svdq_status svdq_pack_weights(int64_t K, int64_t N, const uint16_t* W, const float* act_absmax, float alpha,
                              int32_t rank, int32_t fmt, float* s_out, float* inv_s_out, uint16_t* L1t_out,
                              uint16_t* L2_out, uint8_t* qW_out, void* sW_out, float* R_out) {
  return pack_impl(K, N, W, act_absmax, alpha, rank, fmt, 0, s_out, inv_s_out, L1t_out, L2_out, qW_out, sW_out,
                   R_out, nullptr);
}

svdq_status svdq_pack_weights_refined(int64_t K, int64_t N, const uint16_t* W, const float* act_absmax,
                                      float alpha, int32_t rank, int32_t fmt, int32_t iters, float* s_out,
                                      float* inv_s_out, uint16_t* L1t_out, uint16_t* L2_out, uint8_t* qW_out,
                                      void* sW_out, float* R_out, double* err_out) {
  return pack_impl(K, N, W, act_absmax, alpha, rank, fmt, iters, s_out, inv_s_out, L1t_out, L2_out, qW_out, sW_out,
                   R_out, err_out);
}

svdq_status svdq_concat_lora(int64_t K, int64_t N, const float* s, int32_t rank, const uint16_t* L1t,
                             const uint16_t* L2, int32_t lora_rank, const uint16_t* A, const uint16_t* B,
                             float lora_scale, uint16_t* L1t_out, uint16_t* L2_out) {
  if (K < 1 || N < 1) return fail(SVDQ_EINVAL, "K and N must be >= 1");
  if (rank < 0 || lora_rank < 0) return fail(SVDQ_EINVAL, "ranks must be >= 0");
  if (rank + lora_rank > SVDQ_MAX_RANK)
    return fail(SVDQ_EUNSUPPORTED, "rank + lora_rank exceeds %d", SVDQ_MAX_RANK);
  if (!s || !L1t_out || !L2_out || (rank > 0 && (!L1t || !L2)) || (lora_rank > 0 && (!A || !B)))
    return fail(SVDQ_EINVAL, "required pointer is NULL");
  if (!std::isfinite(lora_scale)) return fail(SVDQ_ENUMERIC, "lora_scale must be finite");
  if (rank > 0) {
    std::memmove(L1t_out, L1t, sizeof(uint16_t) * (size_t)rank * K);
    std::memmove(L2_out, L2, sizeof(uint16_t) * (size_t)rank * N);
  }
  for (int64_t t = 0; t < lora_rank; ++t)
    for (int64_t k = 0; k < K; ++k) {
      const double v = ((double)lora_scale * (double)s[k]) * bf16_to_double(A[k * lora_rank + t]);
      L1t_out[(rank + t) * K + k] = double_to_bf16(v);
    }
  std::memcpy(L2_out + (size_t)rank * N, B, sizeof(uint16_t) * (size_t)lora_rank * N);
  return ok();
}

svdq_status svdq_prepare_lowrank_down(int64_t K, int32_t rank, const uint16_t* L1t, uint16_t* L1f_out) {
  if (K < 64 || K % 64 != 0 || rank < 0) return fail(SVDQ_EINVAL, "need K a positive multiple of 64 and rank >= 0");
  if (rank > SVDQ_MAX_RANK) return fail(SVDQ_EUNSUPPORTED, "rank exceeds %d", SVDQ_MAX_RANK);
  if (rank == 0) return ok();
  if (!L1t || !L1f_out) return fail(SVDQ_EINVAL, "required pointer is NULL");
  const int64_t nt = (rank + 15) / 16;
  for (int64_t c = 0; c < K / 64; ++c)
    for (int64_t t = 0; t < nt; ++t)
      for (int64_t l = 0; l < 64; ++l) {
        const int64_t j = t * 16 + (l & 15), k0 = c * 64 + (l >> 4) * 16;
        uint16_t* dst = L1f_out + ((c * nt + t) * 64 + l) * 16;
        for (int64_t e = 0; e < 16; ++e) dst[e] = j < rank ? L1t[j * K + k0 + e] : (uint16_t)0;
      }
  return ok();
}

svdq_status svdq_prepare_lowrank(int64_t N, int32_t rank, const uint16_t* L2, uint16_t* L2f_out) {
  if (N < 1 || rank < 0) return fail(SVDQ_EINVAL, "need N >= 1 and rank >= 0");
  if (rank > SVDQ_MAX_RANK) return fail(SVDQ_EUNSUPPORTED, "rank exceeds %d", SVDQ_MAX_RANK);
  if (rank == 0) return ok();
  if (!L2 || !L2f_out) return fail(SVDQ_EINVAL, "required pointer is NULL");
  const int64_t S = (rank + 15) / 16, N32 = (N + 31) / 32 * 32;
  for (int64_t n = 0; n < N32; ++n)
    for (int64_t j = 0; j < S * 16; ++j) {
      const int64_t e = ((((n >> 5) * S + (j >> 4)) * 64 + (n & 31) + 32 * ((j >> 3) & 1)) << 3) + (j & 7);
      L2f_out[e] = (j < rank && n < N) ? L2[j * N + n] : (uint16_t)0;
    }
  return ok();
}

svdq_status svdq_prepare_weights(int64_t K, int64_t N, int32_t fmt, const uint8_t* qW, const void* sW,
                                 uint8_t* qW_out, void* sW_out) {
  svdq_status st = check_dims(K, N, fmt);
  if (st != SVDQ_OK) return st;
  if (!qW || !sW || !qW_out || !sW_out) return fail(SVDQ_EINVAL, "required pointer is NULL");
  const int64_t groups = K / group_of(fmt);
  const int64_t Np = (N + 3) / 4 * 4;  // scale rows padded to 4 bytes (fp16 rows: 8)
  if (fmt == SVDQ_NVFP4_G16) {
    // codes: column pairs as for MXFP4; inside each 64-block code k moves to nibble
    // 2 (16 ((k / 8) % 2) + 4 (k / 16)) + k % 8, the lane order of the bf16 matrix core
    const int64_t N2 = N + (N & 1);
    std::memset(qW_out, 0, (size_t)(N2 * (K / 2)));
    for (int64_t n = 0; n < N; ++n)
      for (int64_t k0 = 0; k0 < K; k0 += 64) {
        uint8_t blk[32] = {};
        for (int k = 0; k < 64; ++k) {
          const uint8_t byte = qW[n * (K / 2) + (k0 + k) / 2];
          const uint8_t nib = (k & 1) ? byte >> 4 : byte & 15;
          const int p = 2 * (16 * ((k >> 3) & 1) + 4 * (k >> 4)) + (k & 7);
          blk[p >> 1] |= (uint8_t)(nib << (4 * (p & 1)));
        }
        const int64_t b = k0 / 2;
        std::memcpy(qW_out + (n / 2) * K + (b / 64) * 128 + (n % 2) * 64 + b % 64, blk, 32);
      }
    // scales: [K/64][Np][4], the four groups of a 64-block contiguous per column
    const uint8_t* s8 = static_cast<const uint8_t*>(sW);
    uint8_t* o8 = static_cast<uint8_t*>(sW_out);
    for (int64_t g = 0; g < groups; ++g)
      for (int64_t n = 0; n < Np; ++n) {
        const uint8_t e = n < N ? s8[g * N + n] : (uint8_t)0;
        if (e >= 0x7F) return fail(SVDQ_ENUMERIC, "E4M3 weight scale out of range");
        o8[((g / 4) * Np + n) * 4 + g % 4] = e;
      }
    return ok();
  }
  if (fmt == SVDQ_MXFP4_G32) {
    // codes as stored, columns in pairs (see the INT4 placement below)
    const int64_t N2 = N + (N & 1);
    std::memset(qW_out, 0, (size_t)(N2 * (K / 2)));
    for (int64_t n = 0; n < N; ++n)
      for (int64_t b = 0; b < K / 2; b += 64)
        std::memcpy(qW_out + (n / 2) * K + (b / 64) * 128 + (n % 2) * 64, qW + n * (K / 2) + b, 64);
    const uint8_t* s8 = static_cast<const uint8_t*>(sW);
    uint8_t* o8 = static_cast<uint8_t*>(sW_out);
    for (int64_t g = 0; g < groups; ++g)
      for (int64_t n = 0; n < Np; ++n) o8[g * Np + n] = n < N ? s8[g * N + n] : (uint8_t)127;
    return ok();
  }
  // codes: kernel 2 multiplies INT4 codes as FP6 E2M3 values q / 8 (sign bit 5,
  // exponent 0, mantissa |q|).  A matrix-core operand half holds the 32 codes of one
  // group half as 6-bit fields at bit 6f of six words; field f carries k = 16 (f & 1) +
  // (f >> 1) of the half (the order kernel 1's converter produces).  Bits 3-4 of every
  // field are zero, and the info bits of words 2 and 5 sit exactly on the zero bits of
  // words 0, 1 and 3, 4, so the 32 codes are stored in four words w0..w3:
  //   w0 = f0 | (f2 & Z0), w1 = f1 | (f2 & Z1), w2 = f3 | (f5 & Z0), w3 = f4 | (f5 & Z1)
  // and expanded with masks alone (f0 = w0 & ~Z0, f2 = (w0 & Z0) | (w1 & Z1), ...).
  const uint32_t Z0 = (3u << 3) | (3u << 9) | (3u << 15) | (3u << 21) | (3u << 27);
  const uint32_t Z1 = (3u << 1) | (3u << 7) | (3u << 13) | (3u << 19) | (3u << 25) | (1u << 31);
  // Placement: kernel 2 moves 128 K values (64 bytes of a column) per stage, so the
  // 64-byte segments of columns 2j and 2j+1 for a stage share one 128-byte line:
  // byte b of column n goes to (n / 2) K + (b / 64) 128 + (n % 2) 64 + b % 64.  With N
  // odd, the last line pair's second half (a phantom column) is zero.
  const int64_t rowb = K / 2;
  const int64_t N2 = N + (N & 1);
  std::memset(qW_out, 0, (size_t)(N2 * rowb));
  for (int64_t n = 0; n < N; ++n)
    for (int64_t h0 = 0; h0 < K; h0 += 32) {  // one group half: codes h0 .. h0 + 31
      const uint8_t* src = qW + n * rowb + h0 / 2;
      uint32_t f[6] = {0, 0, 0, 0, 0, 0};
      for (int fi = 0; fi < 32; ++fi) {
        const int k = 16 * (fi & 1) + (fi >> 1);
        const uint32_t nib = (src[k >> 1] >> (4 * (k & 1))) & 0xFu;
        const uint32_t v = (nib & 7u) | ((nib & 8u) << 2);  // sign bit 3 -> field bit 5
        const uint64_t sh = (uint64_t)v << ((6 * fi) & 31);
        f[(6 * fi) >> 5] |= (uint32_t)sh;
        if ((6 * fi & 31) > 26) f[((6 * fi) >> 5) + 1] |= (uint32_t)(sh >> 32);
      }
      const uint32_t w[4] = {f[0] | (f[2] & Z0), f[1] | (f[2] & Z1), f[3] | (f[5] & Z0), f[4] | (f[5] & Z1)};
      const int64_t b = h0 / 2;  // byte of the column
      std::memcpy(qW_out + (n / 2) * K + (b / 64) * 128 + (n % 2) * 64 + b % 64, w, 16);
    }
  // scales: the fp16 bits, [groups][Np], padding 0
  const uint16_t* s16 = static_cast<const uint16_t*>(sW);
  uint16_t* o16 = static_cast<uint16_t*>(sW_out);
  for (int64_t g = 0; g < groups; ++g)
    for (int64_t n = 0; n < Np; ++n) {
      const uint16_t h = n < N ? s16[g * N + n] : (uint16_t)0;
      if (h & 0x8000u) return fail(SVDQ_ENUMERIC, "negative weight scale");
      if (((h >> 10) & 0x1F) == 0x1F) return fail(SVDQ_ENUMERIC, "non-finite weight scale");
      o16[g * Np + n] = h;
    }
  return ok();
}

}  // extern "C"
