// The low-rank up projection as a kernel of its own: Y += lora_act L2, a read and a
// write of the whole output on top of the 4-bit GEMM's own write.
//
// This is the unfused arrangement the SVDQuant review sets against its fused kernels
// (jeonghoonpark.com "SVDQuant" review, section 4.3, Figure 6(a)): the low-rank branch
// run as separate down- and up-projection kernels, which re-read the 16-bit input and
// re-read and re-write the 16-bit output.  The library keeps it as the baseline the fused
// path is measured against; its arithmetic is the fused kernel's low-rank step.
//
// Work split: a block of 4 waves owns a 128 x 128 tile of Y, wave w the 64 x 64 quarter
// (w >> 1, w & 1) as 2 x 2 accumulators of v_mfma_f32_32x32x16_bf16.  lora_act arrives
// as bf16 hi/lo pairs (x = hi + lo to ~2^-17 relative) and L2 as bf16, both in the
// matrix core's fragment order (1 KB per 32-row block and k step); each accumulator
// takes the hi and the lo product, so the branch keeps fp32 accuracy.  Consecutive
// blocks walk along N, so a block's lora_act rows and all of L2f (N * R16 * 2 bytes)
// stay in cache; Y is read and written once.
#include "common.hpp"
#include "kernels.hpp"

namespace svdq {
namespace {

constexpr int UP_BM = 128, UP_BN = 128, UP_THREADS = 256;

// Y[rows r_off.., columns c_off..] += acc for one 32 x 32 accumulator of the tile at
// (m0, n0): lane l32 + 32 kh holds column c_off + l32, rows r_off + 8 (a >> 2) + 4 kh +
// (a & 3).  Rows past the end fall outside the resource's range (loads read zero, stores
// are dropped); columns past N are masked.  The host guarantees 128 * ldy * 4 < 2^32.
__device__ __forceinline__ void add_sub(const v16f& acc, void* Y, int64_t ldy, int ydtype, int64_t m0,
                                        int64_t n0, int64_t rows, int64_t N, int r_off, int c_off, int l32,
                                        int kh) {
  if (n0 + c_off + l32 >= N) return;
  const uint32_t ysz = ydtype == 0 ? 4u : 2u;
  const uint32_t ystep = (uint32_t)ldy * ysz;
  const __amdgpu_buffer_rsrc_t rY = make_rsrc(static_cast<uint8_t*>(Y) + (m0 * ldy + n0) * ysz,
                                              (uint32_t)rows * ystep - (uint32_t)n0 * ysz);
  const uint32_t o = (uint32_t)(r_off + 4 * kh) * ystep + (uint32_t)(c_off + l32) * ysz;
  uint32_t v[16];
  if (ydtype == 0) {
#pragma unroll
    for (int a = 0; a < 16; ++a) v[a] = buf_load4(rY, o + (uint32_t)(8 * (a >> 2) + (a & 3)) * ystep);
#pragma unroll
    for (int a = 0; a < 16; ++a)
      buf_store4(__float_as_uint(__uint_as_float(v[a]) + acc[a]), rY, o + (uint32_t)(8 * (a >> 2) + (a & 3)) * ystep);
  } else {
#pragma unroll
    for (int a = 0; a < 16; ++a) v[a] = buf_load2(rY, o + (uint32_t)(8 * (a >> 2) + (a & 3)) * ystep);
#pragma unroll
    for (int a = 0; a < 16; ++a)
      buf_store2((uint16_t)f32_to_bf16_rne(bf16_lo_to_f32(v[a]) + acc[a]), rY,
                 o + (uint32_t)(8 * (a >> 2) + (a & 3)) * ystep);
  }
}

__global__ __launch_bounds__(UP_THREADS) void k3_lora_up(const uint16_t* __restrict__ lora_act,
                                                         const uint16_t* __restrict__ L2f, int rank, int64_t M,
                                                         int64_t N, void* __restrict__ Y, int64_t ldy, int ydtype,
                                                         uint32_t tiles_n) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, kh = lane >> 5;
  const int64_t m0 = (int64_t)(blockIdx.x / tiles_n) * UP_BM, n0 = (int64_t)(blockIdx.x % tiles_n) * UP_BN;
  const int64_t rowsA = M - m0 < UP_BM ? M - m0 : UP_BM, rowsB = N - n0 < UP_BN ? N - n0 : UP_BN;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  const int R16 = (rank + 15) & ~15;
  // whole 32-row blocks: rows past M are never stored, columns past N are zero in L2f
  const __amdgpu_buffer_rsrc_t rL = make_rsrc(lora_act + m0 * 2 * R16, (uint32_t)(((rowsA + 31) & ~31) * R16 * 4));
  const __amdgpu_buffer_rsrc_t rU = make_rsrc(L2f + n0 * R16, (uint32_t)(((rowsB + 31) & ~31) * R16 * 2));
  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = v16f{};
  for (int k0 = 0; k0 < R16; k0 += 16) {
    v8bf bl[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
      bl[j] = __builtin_bit_cast(v8bf, buf_load16(rU, (uint32_t)(((((wn >> 5) + j) * (R16 >> 4) + (k0 >> 4)) * 64 + lane) * 16)));
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t o = (uint32_t)(((((wm >> 5) + i) * (R16 >> 4) + (k0 >> 4)) * 2 * 64 + lane) * 16);
      const v8bf ah = __builtin_bit_cast(v8bf, buf_load16(rL, o));
      const v8bf al = __builtin_bit_cast(v8bf, buf_load16(rL, o + 64 * 16));
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bl[j], acc[i][j], 0, 0, 0);
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bl[j], acc[i][j], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) add_sub(acc[i][j], Y, ldy, ydtype, m0, n0, rowsA, N, wm + i * 32, wn + j * 32, l32, kh);
}

}  // namespace

hipError_t launch_lora_up(const KernelLayer& L, int64_t M, const void* lora_act, void* Y, int64_t ldy,
                          int ydtype, hipStream_t st) {
  const uint32_t tiles_m = (uint32_t)((M + UP_BM - 1) / UP_BM), tiles_n = (uint32_t)((L.N + UP_BN - 1) / UP_BN);
  hipLaunchKernelGGL(k3_lora_up, dim3(tiles_m * tiles_n), dim3(UP_THREADS), 0, st,
                     static_cast<const uint16_t*>(lora_act), L.L2f, L.rank, M, L.N, Y, ldy, ydtype, tiles_n);
  return hipGetLastError();
}

}  // namespace svdq
