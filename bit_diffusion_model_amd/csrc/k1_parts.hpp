// Per-chunk steps of kernel 1 on one lane's 16 smoothed activations, shared by kernel 1
// (activations from HBM) and by the chained MLP epilogue of kernel 2 (the next layer's
// activations from the tile in LDS).  Lane l holds token l & 15 and the 16 consecutive
// channels 16 (l >> 4) .. +15 of a 64-wide chunk, so one INT4 group (64) spans the lanes
// l, l ^ 16, l ^ 32, l ^ 48.  Every lane of the wave must call these together (they use
// cross-lane operations).
#pragma once
#include "common.hpp"

namespace svdq {

// INT4 quantizer of a group (the review's section 3 equation Q_X = round(X / s_X), s_X =
// max|X| / 7): s = fp16(fp32(a / 7)) with a the group's max |x| (saturating at 65504);
// the fp32 quotient a / 7 is formed as q0 = a * fp32(1/7) corrected by one fma with the
// exact residual a - 7 q0, which gives the correctly rounded quotient for every
// non-negative finite fp32 a (checked exhaustively).  t[i] = round-half-even(x / s)
// exactly: t = x * rcp(s) (v_rcp_f32, within 1 ulp of 1 / s) is within |x / s| 2^-22 of
// the quotient, so rint(t) is the correctly rounded code unless x / s lies within 2^-17
// of a half integer; then (if any lane of the wave has one) the exact residual x - q s
// decides, ties to even.  s = 0 (an all-zero group, or one whose fp16 scale underflows)
// leaves every code 0.  Returns s; t is not clamped.
__device__ __forceinline__ _Float16 int4_quantize16(const float (&xh)[16], float (&t)[16]) {
  float a = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) a = fmaxf(a, fabsf(xh[i]));
  a = wave_max_xor(a, 16);
  a = wave_max_xor(a, 32);
  constexpr float kSeventh = 1.0f / 7.0f;
  const float q0 = a * kSeventh;
  const float a7 = fmaf(fmaf(-q0, 7.0f, a), kSeventh, q0);  // == fp32(a / 7)
  const _Float16 sh = (_Float16)fminf(a7, 65504.0f);
  const float sf = (float)sh;
  const float rcp = sf > 0.0f ? __builtin_amdgcn_rcpf(sf) : 0.0f;
  float dev = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    t[i] = xh[i] * rcp;
    dev = fmaxf(dev, fabsf(t[i] - rintf(t[i])));
  }
  if (__builtin_amdgcn_ballot_w64(dev > 0.49999237f) != 0) {  // 0.5 - 2^-17
    // with s = 0 the codes stay 0: no |x - q s| exceeds an infinite half-scale
    const float hs = sf > 0.0f ? 0.5f * sf : __builtin_inff();
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float q = rintf(t[i]);
      const float e = fmaf(-q, sf, xh[i]);
      const float ae = fabsf(e);
      const int odd = ((int)q) & 1;
      const int away = (int)(ae > hs) | ((int)(ae == hs) & odd);
      t[i] = q + (float)away * copysignf(1.0f, e);
    }
  }
  return sh;
}

// The lane's 16 bytes of the MMA form (FP6 E2M3 operand fields, sign << 5 | |q|, value
// q / 8): the converter writes t / 8 rounded half to even on the E2M3 subnormal grid of
// step 1/8 (the field of round(t)), interleaving its two 16-value inputs field by field,
// so the lanes of quarters 2h, 2h+1 of a group (l and l ^ 16) each convert their 16 codes
// twice, exchange halves with one row swap per word and keep the even fields of the even
// quarter and the odd fields of the odd one: field f of half h holds k = 32 h + 16 (f &
// 1) + (f >> 1).  A half is stored as [w0 w1 w2 w3 | w4 w5 0 0]: the even quarter takes
// word 3 across the pair, then stores words 0-3, the odd quarter words 4-5.  The clamp
// to +-7 only acts for subnormal fp16 scales; code 0 may carry either sign bit.
__device__ __forceinline__ uint4 int4_mma_words(const float (&t)[16], int sub) {
  v16f tc;
#pragma unroll
  for (int i = 0; i < 16; ++i) tc[i] = __builtin_amdgcn_fmed3f(t[i], -7.0f, 7.0f);
  const v6i f6 = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(tc, tc, 8.0f);
  keep_live(tc);
  // bits of the even fields (field 2i at bit 12 i) in words d and d + 3
  constexpr uint32_t EV[3] = {0x3F03F03Fu, 0xF03F03F0u, 0x03F03F03u};
  uint32_t fw[3];
#pragma unroll
  for (int d = 0; d < 3; ++d) {
    // even rows (quarters 0, 2) receive the odd row's word d, odd rows the even row's
    // word d + 3
    const auto r = __builtin_amdgcn_permlane16_swap((uint32_t)f6[d], (uint32_t)f6[d + 3], false, false);
    fw[d] = (r[0] & EV[d]) | (r[1] & ~EV[d]);
  }
  const uint32_t w3 = __builtin_amdgcn_permlane16_swap(fw[0], fw[0], false, false)[1];
  return (sub & 1) ? make_uint4(fw[1], fw[2], 0u, 0u) : make_uint4(fw[0], fw[1], fw[2], w3);
}

typedef __bf16 bf2_t __attribute__((ext_vector_type(2)));

// fp32 pair -> bf16 pair bits, round to nearest even (element a in the low half)
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  const bf2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Down projection step: acc[t] += X_hat (16 tokens x the chunk's 64 channels) L1 (the
// chunk's 64 rows, rank tile t) on v_mfma_f32_16x16x32_bf16, with each fp32 value split
// into a bf16 pair hi + lo (x to ~2^-17) against the same L1 fragment.  Lane l supplies
// MFMA row l & 15 and k-block l >> 4: its first 8 channels go to one MFMA and the next 8
// to a second; LA / LB are the lane's two 16-byte L1 fragments (the same channel order).
template <int NT>
__device__ __forceinline__ void lora_down16(v4f (&acc)[NT > 0 ? NT : 1], const float (&xh)[16],
                                            const uint4 (&LA)[NT > 0 ? NT : 1], const uint4 (&LB)[NT > 0 ? NT : 1]) {
  if constexpr (NT > 0) {
    uint32_t hw[8], lw[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      hw[j] = pk_bf16(xh[2 * j], xh[2 * j + 1]);
      lw[j] = pk_bf16(xh[2 * j] - bf16_lo_to_f32(hw[j]), xh[2 * j + 1] - bf16_hi_to_f32(hw[j]));
    }
    const v8bf a0h = __builtin_bit_cast(v8bf, make_uint4(hw[0], hw[1], hw[2], hw[3]));
    const v8bf a1h = __builtin_bit_cast(v8bf, make_uint4(hw[4], hw[5], hw[6], hw[7]));
    const v8bf a0l = __builtin_bit_cast(v8bf, make_uint4(lw[0], lw[1], lw[2], lw[3]));
    const v8bf a1l = __builtin_bit_cast(v8bf, make_uint4(lw[4], lw[5], lw[6], lw[7]));
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const v8bf bA = __builtin_bit_cast(v8bf, LA[t]), bB = __builtin_bit_cast(v8bf, LB[t]);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0h, bA, acc[t], 0, 0, 0);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1h, bB, acc[t], 0, 0, 0);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0l, bA, acc[t], 0, 0, 0);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1l, bB, acc[t], 0, 0, 0);
    }
  }
}

// The MMA form of a down-projection result v at (token m, rank j): the bf16 pair kernel 2's
// up-projection MFMA consumes, v = hi + lo to ~2^-17 relative, in its fragment order:
// 32-row blocks, k steps of 16, hi then lo (512 elements apart), the 64 lanes' 8 values
// (lane m % 32 + 32 (j / 8 % 2)).  S = R16 / 16.
__device__ __forceinline__ void store_lora_mma(uint16_t* la, int64_t m, int j, int S, float v) {
  const uint32_t hb = f32_to_bf16_rne(v);
  const uint32_t lb = f32_to_bf16_rne(v - __uint_as_float(hb << 16));
  uint16_t* p = la + (((((m >> 5) * S + (j >> 4)) * 2) * 64 + (m & 31) + 32 * ((j >> 3) & 1)) << 3) + (j & 7);
  p[0] = (uint16_t)hb;
  p[512] = (uint16_t)lb;
}

}  // namespace svdq
