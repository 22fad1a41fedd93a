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
  const uint16_t* Ld_hi;
  const uint16_t* Ld_lo;
  const uint16_t* L2t;
  const uint8_t* qW;
  const void* sW;
};

// fp8_codes (INT4 only): write the activation codes as one FP8 E4M3 byte each, [M][K],
// instead of nibble pairs [M][K/2] (the form kernel 2 consumes without expanding).
hipError_t launch_k1(const KernelLayer& L, int64_t M, const uint16_t* X, int64_t ldx, uint8_t* qX,
                     void* sX, float* lora_act, bool fp8_codes, hipStream_t st);

// ydtype: 0 fp32, 1 bf16.  fp8_codes: qX holds FP8 bytes [M][K] (INT4 only).
hipError_t launch_k2(const KernelLayer& L, int64_t M, const uint8_t* qX, const void* sX,
                     const float* lora_act, void* Y, int64_t ldy, int ydtype, bool fp8_codes,
                     hipStream_t st);

hipError_t launch_k2_debug(const KernelLayer& L, int64_t M, const uint8_t* qX, int64_t m0,
                           int64_t n0, int64_t mt, int64_t nt, int32_t* out, hipStream_t st);

}  // namespace svdq
