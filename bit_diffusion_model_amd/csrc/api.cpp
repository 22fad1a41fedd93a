// C ABI: argument validation, error reporting and kernel launches for the device
// entry points declared in include/svdq.h.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/svdq.h"
#include "internal.hpp"
#include "kernels.hpp"

namespace svdq {

static thread_local std::string g_err;

svdq_status fail(svdq_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

svdq_status ok() {
  g_err.clear();
  return SVDQ_OK;
}

static bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int group_of(int fmt) { return fmt == SVDQ_INT4_G64 ? 64 : 32; }

svdq_status check_dims(int64_t K, int64_t N, int32_t fmt) {
  if (fmt != SVDQ_INT4_G64 && fmt != SVDQ_MXFP4_G32)
    return fail(SVDQ_EUNSUPPORTED, "unsupported format %d", (int)fmt);
  if (K < 128 || K % 128 != 0) return fail(SVDQ_EINVAL, "K must be a positive multiple of 128 (got %lld)", (long long)K);
  if (N < 1) return fail(SVDQ_EINVAL, "N must be >= 1 (got %lld)", (long long)N);
  return SVDQ_OK;
}

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
  kl = KernelLayer{L->K, L->N, L->rank, L->fmt, L->inv_s, L->L1f, L->L2f, L->qW, L->sW};
  return SVDQ_OK;
}

static size_t rup(size_t x) { return (x + 255) & ~size_t(255); }

struct WsLayout {
  size_t qx, sx, la, part, total;
};
// The forward path's workspace: the activation side in MMA form (INT4 FP6 operand
// words, 64 bytes per token and group, and an fp16 scale plane; MXFP4 codes in token
// pairs and E8M0 bytes; lora_act as bf16 hi/lo pairs in fragment order, M rounded up to
// 32 rows), then kernel 2's partial tiles.
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
  KernelLayer kl{L->K, L->N, L->rank, L->fmt, nullptr, nullptr, nullptr, nullptr, nullptr};
  w.total = w.part + rup(plan_k2(kl, M, true).bytes);
  return w;
}

}  // namespace svdq

using namespace svdq;

extern "C" {

const char* svdq_last_error(void) { return g_err.c_str(); }

size_t svdq_workspace_bytes(const svdq_layer* layer, int64_t M) {
  if (!layer || M < 0 || check_dims(layer->K, layer->N, layer->fmt) != SVDQ_OK) return 0;
  return ws_layout(layer, M).total;
}

size_t svdq_gemm_workspace_bytes(const svdq_layer* layer, int64_t M, int32_t form) {
  if (!layer || M < 1 || check_dims(layer->K, layer->N, layer->fmt) != SVDQ_OK) return 0;
  KernelLayer kl{layer->K, layer->N, layer->rank, layer->fmt, nullptr, nullptr, nullptr, nullptr, nullptr};
  return plan_k2(kl, M, form == SVDQ_ACT_MMA).bytes;
}

}  // extern "C"

namespace svdq {

static svdq_status check_form(int32_t form) {
  if (form != SVDQ_ACT_PACKED && form != SVDQ_ACT_MMA) return fail(SVDQ_EUNSUPPORTED, "unknown activation form %d", (int)form);
  return SVDQ_OK;
}

static svdq_status run_k1(const svdq_layer* layer, int64_t M, const uint16_t* X, int64_t ldx,
                          int32_t form, uint8_t* qX, void* sX, void* lora_act, void* stream) {
  KernelLayer kl;
  svdq_status st = check_layer(layer, kl);
  if (st != SVDQ_OK) return st;
  if ((st = check_form(form)) != SVDQ_OK) return st;
  if (M < 0) return fail(SVDQ_EINVAL, "M must be >= 0");
  if (M == 0) return ok();
  if (!X || !qX || !sX) return fail(SVDQ_EINVAL, "X, qX and sX must be non-NULL");
  if (kl.rank > 0 && !lora_act) return fail(SVDQ_EINVAL, "lora_act must be non-NULL when rank > 0");
  if (ldx < kl.K || ldx % 8 != 0) return fail(SVDQ_EINVAL, "ldx must be >= K and a multiple of 8");
  if (!aligned(X, 16) || !aligned(qX, 16) || !aligned(sX, 2) || (lora_act && !aligned(lora_act, 16)))
    return fail(SVDQ_EINVAL, "X, qX and lora_act must be 16-byte aligned");
  hipError_t e = launch_k1(kl, M, X, ldx, qX, sX, lora_act, form == SVDQ_ACT_MMA, (hipStream_t)stream);
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
  if (ydtype != SVDQ_F32 && ydtype != SVDQ_BF16) return fail(SVDQ_EUNSUPPORTED, "unsupported output dtype %d", (int)ydtype);
  if (!qX || !sX || !Y) return fail(SVDQ_EINVAL, "qX, sX and Y must be non-NULL");
  if (kl.rank > 0 && !lora_act) return fail(SVDQ_EINVAL, "lora_act must be non-NULL when rank > 0");
  if (ldy < kl.N) return fail(SVDQ_EINVAL, "ldy must be >= N");
  if (ldy >= (int64_t(1) << 23)) return fail(SVDQ_EUNSUPPORTED, "ldy must be < 2^23 elements");
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
  st = run_k1(layer, M, X, ldx, SVDQ_ACT_MMA, qX, sX, la, stream);
  if (st != SVDQ_OK) return st;
  return run_k2(layer, M, SVDQ_ACT_MMA, qX, sX, la, Y, ldy, ydtype, base + w.part, w.total - w.part, stream);
}

svdq_status svdq_linear_forward_unfused(const svdq_layer* layer, int64_t M, const uint16_t* X, int64_t ldx,
                                        void* Y, int64_t ldy, int32_t ydtype, void* workspace,
                                        size_t ws_bytes, void* stream) {
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

svdq_status svdq_debug_group_sums(const svdq_layer* layer, int64_t M, const uint8_t* qX, int64_t m0,
                                  int64_t n0, int64_t mt, int64_t nt, int32_t* out, void* stream) {
  KernelLayer kl;
  svdq_status st = check_layer(layer, kl);
  if (st != SVDQ_OK) return st;
  if (kl.fmt != SVDQ_INT4_G64) return fail(SVDQ_EUNSUPPORTED, "group sums are defined for INT4 only");
  if (!qX || !out) return fail(SVDQ_EINVAL, "qX and out must be non-NULL");
  if (m0 < 0 || n0 < 0 || mt < 1 || nt < 1 || m0 + mt > M || n0 + nt > kl.N)
    return fail(SVDQ_EINVAL, "window out of range");
  if (!aligned(qX, 16)) return fail(SVDQ_EINVAL, "qX must be 16-byte aligned");
  hipError_t e = launch_k2_debug(kl, M, qX, m0, n0, mt, nt, out, (hipStream_t)stream);
  if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return fail(SVDQ_EHIP, "group-sum kernel: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
