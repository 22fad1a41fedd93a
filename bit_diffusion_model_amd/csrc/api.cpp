// C ABI: argument validation, error reporting and kernel launches for the device
// entry points declared in include/svdq.h.
#include <hip/hip_runtime.h>

#include <cstdio>

#include "../../include/svdq.h"
#include "internal.hpp"
#include "kernels.hpp"

namespace svdq {

static bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

static svdq_status check_layer(const svdq_layer* L, KernelLayer& kl) {
  if (!L) return fail(SVDQ_EINVAL, "layer is NULL");
  svdq_status st = check_dims(L->K, L->N, L->fmt);
  if (st != SVDQ_OK) return st;
  if (L->rank < 0 || L->rank > SVDQ_MAX_RANK)
    return fail(SVDQ_EUNSUPPORTED, "rank must be in [0, %d] (got %d)", SVDQ_MAX_RANK, (int)L->rank);
  if (!L->inv_s || !L->qW || !L->sW) return fail(SVDQ_EINVAL, "layer inv_s, qW and sW must be non-NULL");
  if (L->rank > 0 && (!L->L1f || !L->L2f))
    return fail(SVDQ_EINVAL, "layer L1f and L2f must be non-NULL when rank > 0");
  if (!aligned(L->sW, 16)) return fail(SVDQ_EINVAL, "layer sW must be 16-byte aligned");
  if (!aligned(L->inv_s, 16) || !aligned(L->qW, 16) ||
      (L->rank > 0 && (!aligned(L->L1f, 16) || !aligned(L->L2f, 16))))
    return fail(SVDQ_EINVAL, "layer inv_s, qW, L1f and L2f must be 16-byte aligned");
  if (L->fmt == SVDQ_NVFP4_G16 && !(L->tscale_w > 0.f && L->tscale_x > 0.f && L->tscale_w < 3.0e38f &&
                                    L->tscale_x < 3.0e38f))
    return fail(SVDQ_EINVAL, "NVFP4 layer tensor scales must be positive and finite");
  const bool nv = L->fmt == SVDQ_NVFP4_G16;
  kl = KernelLayer{L->K, L->N, L->rank, L->fmt, L->inv_s, L->L1f, L->L2f, L->qW, L->sW, nv ? L->tscale_w : 1.f,
                   nv ? L->tscale_x : 1.f};
  return SVDQ_OK;
}

static size_t rup(size_t x) { return (x + 255) & ~size_t(255); }

struct WsLayout {
  size_t qx, sx, la, part, total;
  int k1parts, k1full;
};
// The forward path's workspace: the activation side in MMA form (INT4 FP6 operand
// words, 64 bytes per token and group, and an fp16 scale plane; MXFP4 codes in token
// pairs and E8M0 bytes; lora_act as bf16 hi/lo pairs in fragment order, M rounded up to
// 32 rows), then one region that holds kernel 1's per-part down-projection sums (when
// it is cut along K) and, after kernel 1's second step has added them, kernel 2's
// partial tiles.
static WsLayout ws_layout(const svdq_layer* L, int64_t M) {
  const bool i4 = L->fmt == SVDQ_INT4_G64;
  WsLayout w;
  w.qx = 0;
  // MXFP4 codes in token pairs: an odd M gets a pair's second row
  w.sx = rup(i4 ? (size_t)M * (size_t)L->K : (size_t)((M + 1) & ~int64_t(1)) * (size_t)(L->K / 2));
  // MMA-form scales: rows padded to Mp = M rounded up to 4; INT4 fp16, MXFP4 E8M0 bytes
  const size_t Mp = ((size_t)M + 3) / 4 * 4;
  w.la = w.sx + rup((size_t)(L->K / group_of(L->fmt)) * Mp * (i4 ? 2 : 1));
  w.part = w.la + rup((size_t)((M + 31) & ~int64_t(31)) * (size_t)((L->rank + 15) / 16 * 16) * 4);
  KernelLayer kl{L->K, L->N, L->rank, L->fmt, nullptr, nullptr, nullptr, nullptr, nullptr, 1.f, 1.f};
  const K1Cut cut = k1_cut(kl, M);
  w.k1parts = cut.parts;
  w.k1full = cut.full;
  const size_t k1b = w.k1parts > 1 ? (size_t)w.k1parts * (size_t)(M - 16 * (int64_t)w.k1full) *
                                         (size_t)((L->rank + 15) / 16 * 16) * 4
                                   : 0;
  const size_t k2b = plan_k2(kl, M, true).bytes;
  w.total = w.part + rup(k1b > k2b ? k1b : k2b);
  return w;
}

}  // namespace svdq

using namespace svdq;

extern "C" {

size_t svdq_workspace_bytes(const svdq_layer* layer, int64_t M) {
  if (!layer || M < 0 || check_dims(layer->K, layer->N, layer->fmt) != SVDQ_OK) return 0;
  return ws_layout(layer, M).total;
}

int32_t svdq_forward_k1_parts(const svdq_layer* layer, int64_t M) {
  if (!layer || M < 0 || check_dims(layer->K, layer->N, layer->fmt) != SVDQ_OK) return 0;
  return ws_layout(layer, M).k1parts;
}

size_t svdq_gemm_workspace_bytes(const svdq_layer* layer, int64_t M, int32_t form) {
  if (!layer || M < 1 || check_dims(layer->K, layer->N, layer->fmt) != SVDQ_OK) return 0;
  KernelLayer kl{layer->K, layer->N, layer->rank, layer->fmt, nullptr, nullptr, nullptr, nullptr, nullptr, 1.f, 1.f};
  return plan_k2(kl, M, form == SVDQ_ACT_MMA).bytes;
}

}  // extern "C"

namespace svdq {

static svdq_status check_form(int32_t form) {
  if (form != SVDQ_ACT_PACKED && form != SVDQ_ACT_MMA) return fail(SVDQ_EUNSUPPORTED, "unknown activation form %d", (int)form);
  return SVDQ_OK;
}

static svdq_status run_k1(const svdq_layer* layer, int64_t M, const uint16_t* X, int64_t ldx,
                          int32_t form, uint8_t* qX, void* sX, void* lora_act, void* stream, int parts = 1,
                          float* part_out = nullptr, int full = 0) {
  KernelLayer kl;
  svdq_status st = check_layer(layer, kl);
  if (st != SVDQ_OK) return st;
  if ((st = check_form(form)) != SVDQ_OK) return st;
  if (M < 0) return fail(SVDQ_EINVAL, "M must be >= 0");
  if (M == 0) return ok();
  if (!X || !qX || !sX) return fail(SVDQ_EINVAL, "X, qX and sX must be non-NULL");
  if (kl.rank > 0 && !lora_act) return fail(SVDQ_EINVAL, "lora_act must be non-NULL when rank > 0");
  if (ldx < kl.K || ldx % 8 != 0) return fail(SVDQ_EINVAL, "ldx must be >= K and a multiple of 8");
  // the scale planes are addressed through 32-bit buffer offsets
  if (M * kl.K >= (int64_t(1) << 35)) return fail(SVDQ_EUNSUPPORTED, "M * K must be < 2^35");
  if (!aligned(X, 16) || !aligned(qX, 16) || !aligned(sX, 2) || (lora_act && !aligned(lora_act, 16)))
    return fail(SVDQ_EINVAL, "X, qX and lora_act must be 16-byte aligned");
  // at rank 0 the cut needs no workspace, so every kernel-1 launch takes it
  if (kl.rank == 0) {
    const K1Cut cut = k1_cut(kl, M);
    parts = cut.parts;
    full = cut.full;
  }
  hipError_t e = launch_k1(kl, M, X, ldx, qX, sX, lora_act, form == SVDQ_ACT_MMA, (hipStream_t)stream, parts,
                           part_out, full);
  if (e != hipSuccess) return fail(SVDQ_EHIP, "kernel 1 launch: %s", hipGetErrorString(e));
  return ok();
}

static svdq_status run_k2(const svdq_layer* layer, int64_t M, int32_t form, const uint8_t* qX,
                          const void* sX, const void* lora_act, void* Y, int64_t ldy,
                          int32_t ydtype, void* workspace, size_t ws_bytes, void* stream) {
  KernelLayer kl;
  svdq_status st = check_layer(layer, kl);
  if (st != SVDQ_OK) return st;
  if ((st = check_form(form)) != SVDQ_OK) return st;
  if (M < 0) return fail(SVDQ_EINVAL, "M must be >= 0");
  if (M == 0) return ok();
  if (ydtype != SVDQ_F32 && ydtype != SVDQ_BF16 && ydtype != SVDQ_BF16_GELU)
    return fail(SVDQ_EUNSUPPORTED, "unsupported output dtype %d", (int)ydtype);
  if (kl.fmt == SVDQ_NVFP4_G16 && form != SVDQ_ACT_MMA)
    return fail(SVDQ_EUNSUPPORTED, "NVFP4 kernel 2 runs on the MMA activation form only");
  if (!qX || !sX || !Y) return fail(SVDQ_EINVAL, "qX, sX and Y must be non-NULL");
  if (kl.rank > 0 && !lora_act) return fail(SVDQ_EINVAL, "lora_act must be non-NULL when rank > 0");
  if (ldy < kl.N) return fail(SVDQ_EINVAL, "ldy must be >= N");
  // the output stores address a tile's rows (up to 256) through a 32-bit range
  if (ldy >= (int64_t(1) << 22)) return fail(SVDQ_EUNSUPPORTED, "ldy must be < 2^22 elements");
  if (!aligned(qX, 16) || !aligned(Y, ydtype == SVDQ_F32 ? 4 : 2) || !aligned(sX, 2) ||
      (lora_act && !aligned(lora_act, 16)))
    return fail(SVDQ_EINVAL, "qX and lora_act must be 16-byte aligned and Y aligned to its element size");
  if (workspace && !aligned(workspace, 256)) return fail(SVDQ_EINVAL, "workspace must be 256-byte aligned");
  hipError_t e = launch_k2(kl, M, qX, sX, lora_act, Y, ldy, ydtype, form == SVDQ_ACT_MMA, workspace,
                           workspace ? ws_bytes : 0, (hipStream_t)stream);
  if (e != hipSuccess) return fail(SVDQ_EHIP, "kernel 2 launch: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace svdq

extern "C" {

svdq_status svdq_quantize_act_lora_down(const svdq_layer* layer, int64_t M, const uint16_t* X,
                                        int64_t ldx, int32_t form, uint8_t* qX, void* sX,
                                        void* lora_act, void* stream) {
  return run_k1(layer, M, X, ldx, form, qX, sX, lora_act, stream);
}

svdq_status svdq_gemm_w4a4_lora_up(const svdq_layer* layer, int64_t M, int32_t form,
                                   const uint8_t* qX, const void* sX, const void* lora_act,
                                   void* Y, int64_t ldy, int32_t ydtype, void* workspace,
                                   size_t ws_bytes, void* stream) {
  return run_k2(layer, M, form, qX, sX, lora_act, Y, ldy, ydtype, workspace, ws_bytes, stream);
}

svdq_status svdq_linear_forward(const svdq_layer* layer, int64_t M, const uint16_t* X, int64_t ldx,
                                void* Y, int64_t ldy, int32_t ydtype, void* workspace,
                                size_t ws_bytes, void* stream) {
  return svdq::linear_forward(layer, M, X, ldx, Y, ldy, ydtype, workspace, ws_bytes, stream);
}

}  // extern "C"

svdq_status svdq::linear_forward(const svdq_layer* layer, int64_t M, const uint16_t* X, int64_t ldx, void* Y,
                                 int64_t ldy, int32_t ydtype, void* workspace, size_t ws_bytes, void* stream) {
  KernelLayer kl;
  svdq_status st = check_layer(layer, kl);
  if (st != SVDQ_OK) return st;
  if (M < 0) return fail(SVDQ_EINVAL, "M must be >= 0");
  if (M == 0) return ok();
  const WsLayout w = ws_layout(layer, M);
  if (!workspace || ws_bytes < w.total) return fail(SVDQ_EINVAL, "workspace too small: need %zu bytes", w.total);
  if (!aligned(workspace, 256)) return fail(SVDQ_EINVAL, "workspace must be 256-byte aligned");
  uint8_t* base = static_cast<uint8_t*>(workspace);
  uint8_t* qX = base + w.qx;
  void* sX = base + w.sx;
  void* la = kl.rank > 0 ? base + w.la : nullptr;
  st = run_k1(layer, M, X, ldx, SVDQ_ACT_MMA, qX, sX, la, stream, w.k1parts,
              reinterpret_cast<float*>(base + w.part), w.k1full);
  if (st != SVDQ_OK) return st;
  return run_k2(layer, M, SVDQ_ACT_MMA, qX, sX, la, Y, ldy, ydtype, base + w.part, w.total - w.part, stream);
}

extern "C" {

svdq_status svdq_linear_forward_unfused(const svdq_layer* layer, int64_t M, const uint16_t* X, int64_t ldx,
                                        void* Y, int64_t ldy, int32_t ydtype, void* workspace,
                                        size_t ws_bytes, void* stream) {
  KernelLayer kl;
  svdq_status st = check_layer(layer, kl);
  if (st != SVDQ_OK) return st;
  if (M < 0) return fail(SVDQ_EINVAL, "M must be >= 0");
  if (M == 0) return ok();
  // the separate up projection adds to Y, which an activation on the output would break
  if (ydtype == SVDQ_BF16_GELU) return fail(SVDQ_EUNSUPPORTED, "the unfused forward has no GELU output");
  const WsLayout w = ws_layout(layer, M);
  if (!workspace || ws_bytes < w.total) return fail(SVDQ_EINVAL, "workspace too small: need %zu bytes", w.total);
  if (!aligned(workspace, 256)) return fail(SVDQ_EINVAL, "workspace must be 256-byte aligned");
  uint8_t* base = static_cast<uint8_t*>(workspace);
  uint8_t* qX = base + w.qx;
  void* sX = base + w.sx;
  void* la = base + w.la;
  svdq_layer l0 = *layer;  // the 4-bit branch alone
  l0.rank = 0;
  st = run_k1(&l0, M, X, ldx, SVDQ_ACT_MMA, qX, sX, nullptr, stream);
  if (st != SVDQ_OK) return st;
  hipError_t e = hipSuccess;
  if (kl.rank > 0 && (e = launch_k1_down(kl, M, X, ldx, la, (hipStream_t)stream)) != hipSuccess)
    return fail(SVDQ_EHIP, "down-projection launch: %s", hipGetErrorString(e));
  st = run_k2(&l0, M, SVDQ_ACT_MMA, qX, sX, nullptr, Y, ldy, ydtype, base + w.part, w.total - w.part, stream);
  if (st != SVDQ_OK) return st;
  if (kl.rank > 0 && (e = launch_lora_up(kl, M, la, Y, ldy, ydtype, (hipStream_t)stream)) != hipSuccess)
    return fail(SVDQ_EHIP, "up-projection launch: %s", hipGetErrorString(e));
  return ok();
}

svdq_status svdq_w4a16_gemm(int64_t M, int64_t K, int64_t N, const uint16_t* X, int64_t ldx, const uint8_t* qW,
                            const uint16_t* sW, void* Y, int64_t ldy, int32_t ydtype, void* stream) {
  if (M < 0) return fail(SVDQ_EINVAL, "M must be >= 0");
  if (K < 64 || K % 64 != 0 || N < 1) return fail(SVDQ_EINVAL, "K must be a positive multiple of 64 and N >= 1");
  if (M == 0) return ok();
  if (!X || !qW || !sW || !Y) return fail(SVDQ_EINVAL, "X, qW, sW and Y must be non-NULL");
  if (ydtype != SVDQ_F32 && ydtype != SVDQ_BF16) return fail(SVDQ_EUNSUPPORTED, "unsupported output dtype %d", (int)ydtype);
  if (ldx < K || ldx % 8 != 0) return fail(SVDQ_EINVAL, "ldx must be >= K and a multiple of 8");
  if (ldy < N) return fail(SVDQ_EINVAL, "ldy must be >= N");
  // a tile's rows of X and Y and the scale plane are addressed through 32-bit offsets
  if (ldx >= (int64_t(1) << 22) || ldy >= (int64_t(1) << 22) || (K / 64) * N >= (int64_t(1) << 31))
    return fail(SVDQ_EUNSUPPORTED, "ldx and ldy must be < 2^22 and K / 64 * N < 2^31");
  if (!aligned(X, 16) || !aligned(qW, 16) || !aligned(sW, 2) || !aligned(Y, ydtype == SVDQ_F32 ? 4 : 2))
    return fail(SVDQ_EINVAL, "X and qW must be 16-byte aligned, sW and Y aligned to their element size");
  hipError_t e = launch_w4a16(M, K, N, X, ldx, qW, sW, Y, ldy, ydtype, (hipStream_t)stream);
  if (e != hipSuccess) return fail(SVDQ_EHIP, "weight-only kernel launch: %s", hipGetErrorString(e));
  return ok();
}

svdq_status svdq_debug_group_sums(const svdq_layer* layer, int64_t M, int32_t form, const uint8_t* qX,
                                  int64_t m0, int64_t n0, int64_t mt, int64_t nt, int32_t* out, void* stream) {
  KernelLayer kl;
  svdq_status st = check_layer(layer, kl);
  if (st != SVDQ_OK) return st;
  if (kl.fmt != SVDQ_INT4_G64) return fail(SVDQ_EUNSUPPORTED, "group sums are defined for INT4 only");
  if ((st = check_form(form)) != SVDQ_OK) return st;
  if (!qX || !out) return fail(SVDQ_EINVAL, "qX and out must be non-NULL");
  if (m0 < 0 || n0 < 0 || mt < 1 || nt < 1 || m0 + mt > M || n0 + nt > kl.N)
    return fail(SVDQ_EINVAL, "window out of range");
  if (!aligned(qX, 16)) return fail(SVDQ_EINVAL, "qX must be 16-byte aligned");
  hipError_t e = launch_k2_debug(kl, M, qX, form == SVDQ_ACT_MMA, m0, n0, mt, nt, out, (hipStream_t)stream);
  if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return fail(SVDQ_EHIP, "group-sum kernel: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"

// ---------------------------------------------------------------------------------------
// The chained MLP pair (fc1, GELU, fc2)

namespace svdq {

static svdq_status check_pair(const svdq_layer* fc1, const svdq_layer* fc2, KernelLayer& k1, KernelLayer& k2,
                              bool chained) {
  svdq_status st = check_layer(fc1, k1);
  if (st != SVDQ_OK) return st;
  if ((st = check_layer(fc2, k2)) != SVDQ_OK) return st;
  if (k1.N != k2.K) return fail(SVDQ_EINVAL, "fc1's N (%lld) must equal fc2's K (%lld)", (long long)k1.N, (long long)k2.K);
  if (chained && (k1.fmt != SVDQ_INT4_G64 || k2.fmt != SVDQ_INT4_G64))
    return fail(SVDQ_EUNSUPPORTED, "the chained MLP pair runs INT4 layers");
  return SVDQ_OK;
}

static size_t part_bytes(const svdq_layer* fc1, const svdq_layer* fc2, int64_t M) {
  return (size_t)(fc1->N / 128) * (size_t)M * (size_t)((fc2->rank + 15) / 16 * 16) * sizeof(float);
}

struct MlpLayout {
  WsLayout w1, w2;
  size_t a1, part, g, fw, total;
};
// chained: [fc2's forward workspace: its activation side, then its kernel 2's partial
// tiles] [fc1's activation side] [the down-projection partials]; separate: [G bf16
// M x N1] [one forward workspace, fc1's then fc2's]
static MlpLayout mlp_layout(const svdq_layer* fc1, const svdq_layer* fc2, int64_t M, int32_t mode) {
  MlpLayout L{};
  L.w1 = ws_layout(fc1, M);
  L.w2 = ws_layout(fc2, M);
  if (mode == SVDQ_MLP_CHAINED) {
    L.a1 = L.w2.total;
    L.part = L.a1 + rup(L.w1.part);
    L.total = L.part + rup(part_bytes(fc1, fc2, M));
  } else {
    L.g = 0;
    L.fw = rup((size_t)M * (size_t)fc1->N * 2);
    L.total = L.fw + (L.w1.total > L.w2.total ? L.w1.total : L.w2.total);
  }
  return L;
}

static svdq_status run_chain_gemm(const svdq_layer* fc1, const svdq_layer* fc2, int64_t M, const uint8_t* qX,
                                  const void* sX, const void* lora_act, uint8_t* qX2, void* sX2, float* lora_part,
                                  uint16_t* hidden, int64_t ldh, void* stream) {
  KernelLayer k1, k2;
  svdq_status st = check_pair(fc1, fc2, k1, k2, true);
  if (st != SVDQ_OK) return st;
  if (M < 0) return fail(SVDQ_EINVAL, "M must be >= 0");
  if (M == 0) return ok();
  if (!qX || !sX || !qX2 || !sX2) return fail(SVDQ_EINVAL, "qX, sX, qX2 and sX2 must be non-NULL");
  if (k1.rank > 0 && !lora_act) return fail(SVDQ_EINVAL, "lora_act must be non-NULL when fc1's rank > 0");
  if (k2.rank > 0 && !lora_part) return fail(SVDQ_EINVAL, "lora_part must be non-NULL when fc2's rank > 0");
  if (hidden && (ldh < k1.N || ldh % 8 != 0 || !aligned(hidden, 16)))
    return fail(SVDQ_EINVAL, "hidden needs ldh >= fc1's N, ldh %% 8 == 0 and 16-byte alignment");
  if (!aligned(qX, 16) || !aligned(qX2, 16) || !aligned(sX, 2) || !aligned(sX2, 2) ||
      (lora_act && !aligned(lora_act, 16)) || (lora_part && !aligned(lora_part, 16)))
    return fail(SVDQ_EINVAL, "qX, qX2, lora_act and lora_part must be 16-byte aligned");
  hipError_t e = launch_k2_chain(k1, k2, M, qX, sX, lora_act, qX2, sX2, lora_part, hidden, ldh, (hipStream_t)stream);
  if (e != hipSuccess) return fail(SVDQ_EHIP, "chained kernel 2 launch: %s", hipGetErrorString(e));
  return ok();
}

static svdq_status run_chain_reduce(const svdq_layer* fc1, const svdq_layer* fc2, int64_t M, const float* lora_part,
                                    void* lora_act2, void* stream) {
  KernelLayer k1, k2;
  svdq_status st = check_pair(fc1, fc2, k1, k2, true);
  if (st != SVDQ_OK) return st;
  if (M < 0) return fail(SVDQ_EINVAL, "M must be >= 0");
  if (M == 0 || k2.rank == 0) return ok();
  if (!lora_part || !lora_act2) return fail(SVDQ_EINVAL, "lora_part and lora_act2 must be non-NULL");
  if (!aligned(lora_act2, 16)) return fail(SVDQ_EINVAL, "lora_act2 must be 16-byte aligned");
  hipError_t e = launch_lora_reduce(k1, k2, M, lora_part, lora_act2, (hipStream_t)stream);
  if (e != hipSuccess) return fail(SVDQ_EHIP, "partial-sum launch: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace svdq

extern "C" {

svdq_status svdq_mlp_chain_gemm(const svdq_layer* fc1, const svdq_layer* fc2, int64_t M, const uint8_t* qX,
                                const void* sX, const void* lora_act, uint8_t* qX2, void* sX2, float* lora_part,
                                uint16_t* hidden, int64_t ldh, void* stream) {
  return run_chain_gemm(fc1, fc2, M, qX, sX, lora_act, qX2, sX2, lora_part, hidden, ldh, stream);
}

svdq_status svdq_mlp_chain_reduce(const svdq_layer* fc1, const svdq_layer* fc2, int64_t M, const float* lora_part,
                                  void* lora_act2, void* stream) {
  return run_chain_reduce(fc1, fc2, M, lora_part, lora_act2, stream);
}

size_t svdq_mlp_workspace_bytes(const svdq_layer* fc1, const svdq_layer* fc2, int64_t M, int32_t mode) {
  if (!fc1 || !fc2 || M < 0 || (mode != SVDQ_MLP_CHAINED && mode != SVDQ_MLP_SEPARATE)) return 0;
  if (check_dims(fc1->K, fc1->N, fc1->fmt) != SVDQ_OK || check_dims(fc2->K, fc2->N, fc2->fmt) != SVDQ_OK) return 0;
  return mlp_layout(fc1, fc2, M, mode).total;
}

svdq_status svdq_mlp_forward(const svdq_layer* fc1, const svdq_layer* fc2, int64_t M, const uint16_t* X,
                             int64_t ldx, void* Y, int64_t ldy, int32_t ydtype, int32_t mode, void* workspace,
                             size_t ws_bytes, void* stream) {
  if (mode != SVDQ_MLP_CHAINED && mode != SVDQ_MLP_SEPARATE) return fail(SVDQ_EUNSUPPORTED, "unknown MLP mode %d", (int)mode);
  KernelLayer k1, k2;
  svdq_status st = check_pair(fc1, fc2, k1, k2, mode == SVDQ_MLP_CHAINED);
  if (st != SVDQ_OK) return st;
  if (M < 0) return fail(SVDQ_EINVAL, "M must be >= 0");
  if (M == 0) return ok();
  const MlpLayout L = mlp_layout(fc1, fc2, M, mode);
  if (!workspace || ws_bytes < L.total) return fail(SVDQ_EINVAL, "workspace too small: need %zu bytes", L.total);
  if (!aligned(workspace, 256)) return fail(SVDQ_EINVAL, "workspace must be 256-byte aligned");
  uint8_t* base = static_cast<uint8_t*>(workspace);
  if (mode == SVDQ_MLP_SEPARATE) {
    uint16_t* G = reinterpret_cast<uint16_t*>(base + L.g);
    st = svdq::linear_forward(fc1, M, X, ldx, G, k1.N, SVDQ_BF16_GELU, base + L.fw, L.total - L.fw, stream);
    if (st != SVDQ_OK) return st;
    return svdq::linear_forward(fc2, M, G, k1.N, Y, ldy, ydtype, base + L.fw, L.total - L.fw, stream);
  }
  uint8_t* a1 = base + L.a1;
  uint8_t* qX1 = a1 + L.w1.qx;
  void* sX1 = a1 + L.w1.sx;
  void* la1 = k1.rank > 0 ? a1 + L.w1.la : nullptr;
  uint8_t* qX2 = base + L.w2.qx;
  void* sX2 = base + L.w2.sx;
  void* la2 = k2.rank > 0 ? base + L.w2.la : nullptr;
  float* part = k2.rank > 0 ? reinterpret_cast<float*>(base + L.part) : nullptr;
  st = run_k1(fc1, M, X, ldx, SVDQ_ACT_MMA, qX1, sX1, la1, stream);
  if (st != SVDQ_OK) return st;
  st = run_chain_gemm(fc1, fc2, M, qX1, sX1, la1, qX2, sX2, part, nullptr, 0, stream);
  if (st != SVDQ_OK) return st;
  st = run_chain_reduce(fc1, fc2, M, part, la2, stream);
  if (st != SVDQ_OK) return st;
  return run_k2(fc2, M, SVDQ_ACT_MMA, qX2, sX2, la2, Y, ldy, ydtype, base + L.w2.part, L.w2.total - L.w2.part, stream);
}

}  // extern "C"
