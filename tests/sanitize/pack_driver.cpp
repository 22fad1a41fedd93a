// Host-side driver for the sanitizer builds of the library's host code (pack.cpp,
// status.cpp): every host entry point of include/svdq.h on small seeded inputs, with
// several pack threads, plus the error paths.  Exits non-zero on a wrong status or a
// broken invariant; the sanitizers report memory errors, undefined behaviour and data
// races on their own.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

#include "../../include/svdq.h"

static int failures = 0;
#define EXPECT(c)                                                        \
  do {                                                                   \
    if (!(c)) {                                                          \
      std::fprintf(stderr, "FAILED %s at line %d: %s\n", #c, __LINE__, svdq_last_error()); \
      ++failures;                                                        \
    }                                                                    \
  } while (0)

static uint16_t bf16_of(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

struct Pack {
  std::vector<float> s, inv, R;
  std::vector<uint16_t> L1t, L2;
  std::vector<uint8_t> qW, sW;
  std::vector<double> err;
};

static Pack alloc(int64_t K, int64_t N, int rank, int fmt, int iters) {
  Pack p;
  size_t qb = 0, sb = 0;
  EXPECT(svdq_weight_sizes(K, N, fmt, &qb, &sb) == SVDQ_OK);
  p.s.resize(K);
  p.inv.resize(K);
  p.R.resize((size_t)K * N);
  p.L1t.resize((size_t)rank * K + 1);
  p.L2.resize((size_t)rank * N + 1);
  p.qW.resize(qb);
  p.sW.resize(sb);
  p.err.resize(iters + 1);
  return p;
}

int main() {
  std::mt19937 rng(7);
  std::normal_distribution<float> nd(0.f, 1.f);
  const int64_t M = 48, K = 256, N = 200;
  std::vector<uint16_t> X((size_t)M * K), W((size_t)K * N);
  for (auto& v : X) v = bf16_of(nd(rng));
  for (int64_t m = 0; m < M; ++m) X[(size_t)m * K + 5] = bf16_of(30.f * nd(rng));  // an outlier channel
  for (auto& v : W) v = bf16_of(nd(rng));
  std::vector<float> a(K);
  EXPECT(svdq_act_absmax(M, K, X.data(), K, a.data()) == SVDQ_OK);

  for (int fmt = 0; fmt < 3; ++fmt) {  // INT4, MXFP4, NVFP4
    for (int rank : {0, 16}) {
      Pack p = alloc(K, N, rank, fmt, 0);
      EXPECT(svdq_pack_weights(K, N, W.data(), a.data(), 0.5f, rank, fmt, p.s.data(), p.inv.data(), p.L1t.data(),
                               p.L2.data(), p.qW.data(), p.sW.data(), p.R.data()) == SVDQ_OK);
      // refinement: iterate 0 is the plain pack, the kept iterate has the smallest error
      Pack q = alloc(K, N, rank, fmt, 2);
      EXPECT(svdq_pack_weights_refined(K, N, W.data(), a.data(), 0.5f, rank, fmt, 2, q.s.data(), q.inv.data(),
                                       q.L1t.data(), q.L2.data(), q.qW.data(), q.sW.data(), q.R.data(),
                                       q.err.data()) == SVDQ_OK);
      Pack z = alloc(K, N, rank, fmt, 0);
      EXPECT(svdq_pack_weights_refined(K, N, W.data(), a.data(), 0.5f, rank, fmt, 0, z.s.data(), z.inv.data(),
                                       z.L1t.data(), z.L2.data(), z.qW.data(), z.sW.data(), z.R.data(),
                                       z.err.data()) == SVDQ_OK);
      EXPECT(z.qW == p.qW && z.sW == p.sW && z.L1t == p.L1t && z.L2 == p.L2);
      EXPECT(q.err[0] >= q.err[1] || q.err[0] >= q.err[2] || (q.qW == p.qW && q.L1t == p.L1t));
      // the quantizer alone on the pack's residual gives its codes
      std::vector<uint8_t> qW2(p.qW.size()), sW2(p.sW.size());
      EXPECT(svdq_quantize_weights(K, N, p.R.data(), fmt, qW2.data(), sW2.data()) == SVDQ_OK);
      if (fmt == 2) {  // NVFP4: the quantizer alone writes the activations' tensor scale as 1
        const size_t n = sW2.size();
        float sx = 0.f;
        std::memcpy(&sx, sW2.data() + n - 4, 4);
        EXPECT(qW2 == p.qW && std::memcmp(sW2.data(), p.sW.data(), n - 4) == 0 && sx == 1.0f);
      } else {
        EXPECT(qW2 == p.qW && sW2 == p.sW);
      }
      // device layouts
      // scale layouts: INT4 fp16 [K/64][Np], MXFP4 E8M0 [K/32][Np], NVFP4 E4M3 [K/64][Np][4]
      const size_t Np = (size_t)(N + 3) / 4 * 4;
      const size_t sbytes = fmt == 0 ? (size_t)(K / 64) * Np * 2 : fmt == 1 ? (size_t)(K / 32) * Np : (size_t)(K / 16) * Np;
      std::vector<uint8_t> qo((size_t)(N + 1) / 2 * 2 * (K / 2)), so(sbytes);
      EXPECT(svdq_prepare_weights(K, N, fmt, p.qW.data(), p.sW.data(), qo.data(), so.data()) == SVDQ_OK);
      if (rank) {
        const int R16 = (rank + 15) / 16 * 16;
        std::vector<uint16_t> L1f((size_t)R16 * K), L2f((size_t)(N + 31) / 32 * 32 * R16);
        EXPECT(svdq_prepare_lowrank_down(K, rank, p.L1t.data(), L1f.data()) == SVDQ_OK);
        EXPECT(svdq_prepare_lowrank(N, rank, p.L2.data(), L2f.data()) == SVDQ_OK);
        // LoRA fold (rank + 8)
        const int lr = 8;
        std::vector<uint16_t> A((size_t)K * lr), B((size_t)lr * N);
        for (auto& v : A) v = bf16_of(0.02f * nd(rng));
        for (auto& v : B) v = bf16_of(0.02f * nd(rng));
        std::vector<uint16_t> L1o((size_t)(rank + lr) * K), L2o((size_t)(rank + lr) * N);
        EXPECT(svdq_concat_lora(K, N, p.s.data(), rank, p.L1t.data(), p.L2.data(), lr, A.data(), B.data(), 1.0f,
                                L1o.data(), L2o.data()) == SVDQ_OK);
        EXPECT(std::memcmp(L1o.data(), p.L1t.data(), (size_t)rank * K * 2) == 0);
      }
    }
  }
  // error paths: documented status codes, no crash
  Pack p = alloc(K, N, 8, 0, 0);
  EXPECT(svdq_pack_weights(K, N, nullptr, a.data(), 0.5f, 8, 0, p.s.data(), p.inv.data(), p.L1t.data(), p.L2.data(),
                           p.qW.data(), p.sW.data(), nullptr) == SVDQ_EINVAL);
  EXPECT(svdq_pack_weights(100, N, W.data(), a.data(), 0.5f, 8, 0, p.s.data(), p.inv.data(), p.L1t.data(),
                           p.L2.data(), p.qW.data(), p.sW.data(), nullptr) == SVDQ_EINVAL);
  EXPECT(svdq_pack_weights(K, N, W.data(), a.data(), 1.5f, 8, 0, p.s.data(), p.inv.data(), p.L1t.data(), p.L2.data(),
                           p.qW.data(), p.sW.data(), nullptr) == SVDQ_EINVAL);
  EXPECT(svdq_pack_weights(K, N, W.data(), a.data(), 0.5f, 8, 9, p.s.data(), p.inv.data(), p.L1t.data(), p.L2.data(),
                           p.qW.data(), p.sW.data(), nullptr) == SVDQ_EUNSUPPORTED);
  std::vector<uint16_t> Wbad(W);
  Wbad[17] = 0x7FC0;  // NaN
  EXPECT(svdq_pack_weights(K, N, Wbad.data(), a.data(), 0.5f, 8, 0, p.s.data(), p.inv.data(), p.L1t.data(),
                           p.L2.data(), p.qW.data(), p.sW.data(), nullptr) == SVDQ_ENUMERIC);
  EXPECT(std::strlen(svdq_last_error()) > 0);
  EXPECT(svdq_act_absmax(0, K, X.data(), K, a.data()) == SVDQ_EINVAL);
  std::printf("%s (%d failures)\n", failures ? "FAILED" : "ok", failures);
  return failures ? 1 : 0;
}
