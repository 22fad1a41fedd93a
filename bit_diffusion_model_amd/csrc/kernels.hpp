// Internal launch interface between the C ABI (api.cpp) and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace svdq {

struct KernelLayer {
  int64_t K, N;
  int rank;
  int fmt;  // 0 INT4 g64, 1 MXFP4 g32
  const float* inv_s;
  const uint16_t* L1f;  // kernel 1's fragment order (svdq_prepare_lowrank_down)
  const uint16_t* L2f;  // kernel 2's fragment order (svdq_prepare_lowrank)
  const uint8_t* qW;
  const void* sW;
};

// mma: the activation side in the matrix-core operand form (INT4 FP6 operand words,
// fp16 scales; lora_act as bf16 hi/lo pairs in fragment order) instead of the packed
// storage form (4-bit codes [M][K/2], fp16 / E8M0 scales, fp32 lora_act).
hipError_t launch_k1(const KernelLayer& L, int64_t M, const uint16_t* X, int64_t ldx, uint8_t* qX,
                     void* sX, void* lora_act, bool mma, hipStream_t st);

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

// ydtype: 0 fp32, 1 bf16.  mma: as for launch_k1.  workspace (device, may be NULL): used
// for the split when it holds plan_k2's bytes; otherwise every tile is computed whole.
hipError_t launch_k2(const KernelLayer& L, int64_t M, const uint8_t* qX, const void* sX,
                     const void* lora_act, void* Y, int64_t ldy, int ydtype, bool mma,
                     void* workspace, size_t ws_bytes, hipStream_t st);

hipError_t launch_k2_debug(const KernelLayer& L, int64_t M, const uint8_t* qX, int64_t m0,
                           int64_t n0, int64_t mt, int64_t nt, int32_t* out, hipStream_t st);

}  // namespace svdq
