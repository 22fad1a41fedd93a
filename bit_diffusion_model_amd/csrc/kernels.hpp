// Internal launch interface between the C ABI (api.cpp) and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace svdq {

struct KernelLayer {
  int64_t K, N;
  int rank;
  int fmt;  // 0 INT4 g64, 1 MXFP4 g32, 2 NVFP4 g16
  const float* inv_s;
  const uint16_t* L1f;  // kernel 1's fragment order (svdq_prepare_lowrank_down)
  const uint16_t* L2f;  // kernel 2's fragment order (svdq_prepare_lowrank)
  const uint8_t* qW;
  const void* sW;
  float tscale_w, tscale_x;  // NVFP4 tensor scales (1 otherwise)
};

// mma: the activation side in the matrix-core operand form (INT4 FP6 operand words,
// fp16 scales; lora_act as bf16 hi/lo pairs in fragment order) instead of the packed
// storage form (4-bit codes [M][K/2], fp16 / E8M0 scales, fp32 lora_act).
// parts > 1 (with part_out, device, parts * (M - 16 full) * R16 fp32, R16 = rank rounded
// up to 16; not needed at rank 0): the first `full` blocks of 16 tokens run over all of K,
// and the chunks along K of every later block of 16 tokens are cut into `parts` ranges,
// one block per range, whose fp32 down-projection sums are added in part order by a second
// kernel (codes and scales are the same as unsplit; lora_act differs only in the order of
// its fp32 additions).
hipError_t launch_k1(const KernelLayer& L, int64_t M, const uint16_t* X, int64_t ldx, uint8_t* qX,
                     void* sX, void* lora_act, bool mma, hipStream_t st, int parts = 1, float* part_out = nullptr,
                     int full = 0);
// How the forward cuts kernel 1: blocks [0, full) whole, the rest in `parts` K ranges each
// (parts == 1: one pass).
struct K1Cut {
  int full, parts;
};
K1Cut k1_cut(const KernelLayer& L, int64_t M);
int k1_parts(const KernelLayer& L, int64_t M);

// The unfused baseline's two low-rank passes: lora_act = X_hat L1 alone (a second read
// of X; MMA-form lora_act), and Y += lora_act L2 (a read and a write of Y).
hipError_t launch_k1_down(const KernelLayer& L, int64_t M, const uint16_t* X, int64_t ldx, void* lora_act,
                          hipStream_t st);
hipError_t launch_lora_up(const KernelLayer& L, int64_t M, const void* lora_act, void* Y, int64_t ldy,
                          int ydtype, hipStream_t st);

// Work split of kernel 2 on the current device: tiles [0, full) whole, the remaining
// tiles (those of a last, partly filled round of resident blocks) cut into `split` parts
// along K whose fp32 partial tiles take `bytes` of workspace.
struct K2Plan {
  uint32_t tiles_m, tiles_n, full, split;
  size_t bytes;
};
K2Plan plan_k2(const KernelLayer& L, int64_t M, bool mma);

// ydtype: 0 fp32, 1 bf16, 2 bf16 of GELU(y).  mma: as for launch_k1.  workspace (device, may be NULL): used
// for the split when it holds plan_k2's bytes; otherwise every tile is computed whole.
hipError_t launch_k2(const KernelLayer& L, int64_t M, const uint8_t* qX, const void* sX,
                     const void* lora_act, void* Y, int64_t ldy, int ydtype, bool mma,
                     void* workspace, size_t ws_bytes, hipStream_t st);

// The chained MLP pair, INT4: fc1's kernel 2 (MMA activation form, whole tiles) with
// fc2's kernel 1 in its epilogue.  Writes fc2's MMA-form codes qX2 [M][K2] and fp16
// scales sX2 [K2/64][Mp], the down-projection partials part [K2/128][M][R16(fc2)] and,
// when hidden is non-NULL, G = bf16(GELU(H)) [M][ldh].  K2 = L1.N = L2.K.
hipError_t launch_k2_chain(const KernelLayer& L1, const KernelLayer& L2, int64_t M, const uint8_t* qX, const void* sX,
                           const void* lora_act, uint8_t* qX2, void* sX2, float* part, uint16_t* hidden, int64_t ldh,
                           hipStream_t st);
// fc2's lora_act (MMA form) = the sum of the partials over the K2/128 column tiles, in order.
hipError_t launch_lora_reduce(const KernelLayer& L1, const KernelLayer& L2, int64_t M, const float* part, void* la2,
                              hipStream_t st);

// Exact INT4 group sums of a window.  mma: the forward's streamed kernel on MMA-form
// codes (its own schedule); otherwise the packed-form kernel.
hipError_t launch_k2_debug(const KernelLayer& L, int64_t M, const uint8_t* qX, bool mma, int64_t m0,
                           int64_t n0, int64_t mt, int64_t nt, int32_t* out, hipStream_t st);

// The 4-bit weight-only baseline: Y = X bf16(s_W q_W) on the bf16 matrix core.  X bf16
// [M][ldx]; qW storage-form INT4 codes [N][K/2]; sW fp16 [K/64][N]; ydtype 0 fp32, 1 bf16.
hipError_t launch_w4a16(int64_t M, int64_t K, int64_t N, const uint16_t* X, int64_t ldx, const uint8_t* qW,
                        const uint16_t* sW, void* Y, int64_t ldy, int ydtype, hipStream_t st);

}  // namespace svdq
