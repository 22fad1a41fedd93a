// Kernel 1: smoothing + per-group 4-bit quantization + low-rank down projection, in
// one pass over the activations.
//
// Method: the runtime half of the smoothing equation X_hat = X diag(s)^-1
// (ch3chohch3.github.io, "从 Smooth Quant 到 SVD Quant", section "Smooth Quant（W8A8）"),
// the quantizer Q_X = round(X_hat / s_X), s_X = max|X_hat| / q_max per group
// (jeonghoonpark.com "SVDQuant" review, section 3), and the down projection X_hat L1
// fused into the quantization kernel so both share one read of X (review, section 4.3,
// Figure 6(b)).  Activation scales are computed online (ch3chohch3 post, "量化方案").
//
// Work split: a block of 4 waves owns 16 consecutive tokens.  The K dimension is cut
// into 64-wide chunks; wave w takes chunks w, w+4, ...  Inside a chunk, lane l holds
// token (l & 15) and the 16 consecutive channels 16 * (l >> 4) .. +15 (two 16-byte
// loads of X).  One INT4 group (64) is therefore spread over the 4 lanes l, l^16,
// l^32, l^48; one FP4 group (32) over lanes l, l^16.
//
// Down projection: X_hat L1 = X (diag(inv_s) L1).  The fold of inv_s into L1 is done
// offline and stored as a bf16 hi/lo pair (Ld_hi + Ld_lo), so the raw bf16 X is the
// MFMA A operand with no conversion.  v_mfma_f32_16x16x32_bf16: lane l supplies row
// l & 15 and k-block l >> 4; we feed the lane's first 8 channels to one MFMA and the
// next 8 to a second, and the B operand (Ld rows, contiguous along K) uses the same
// channel order.  Partial sums of the 4 waves are added through LDS at the end.
#include "common.hpp"
#include "kernels.hpp"

namespace svdq {

template <int FMT, int NT>
__global__ __launch_bounds__(256) void k1_quant_lora_down(
    const uint16_t* __restrict__ X, int64_t ldx, int64_t M, int64_t K,
    const float* __restrict__ inv_s, const uint16_t* __restrict__ Ldh,
    const uint16_t* __restrict__ Ldl, int rank, uint8_t* __restrict__ qX,
    void* __restrict__ sXv, float* __restrict__ lora_act) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r16 = lane & 15;
  const int sub = lane >> 4;
  const int64_t row = (int64_t)blockIdx.x * 16 + r16;
  const bool row_ok = row < M;
  const int nchunks = (int)(K >> 6);

  v4f acc[NT > 0 ? NT : 1];
#pragma unroll
  for (int t = 0; t < (NT > 0 ? NT : 1); ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int c = wave; c < nchunks; c += 4) {
    const int64_t k0 = (int64_t)c * 64 + sub * 16;
    uint4 xa = make_uint4(0, 0, 0, 0), xb = make_uint4(0, 0, 0, 0);
    if (row_ok) {
      const uint4* px = reinterpret_cast<const uint4*>(X + row * ldx + k0);
      xa = px[0];
      xb = px[1];
    }
    const float4* ps = reinterpret_cast<const float4*>(inv_s + k0);
    float4 s0 = ps[0], s1 = ps[1], s2 = ps[2], s3 = ps[3];
    const uint32_t xw[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
    const float sv[16] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w,
                          s2.x, s2.y, s2.z, s2.w, s3.x, s3.y, s3.z, s3.w};
    float xh[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      xh[2 * i] = bf16_lo_to_f32(xw[i]) * sv[2 * i];
      xh[2 * i + 1] = bf16_hi_to_f32(xw[i]) * sv[2 * i + 1];
    }
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) a = fmaxf(a, fabsf(xh[i]));
    a = wave_max_xor(a, 16);

    uint32_t nib[16];
    if constexpr (FMT == 0) {
      // INT4: s = fp16(fp32(a / 7)), saturating; q = round-half-even(x / s) exactly.
      a = wave_max_xor(a, 32);
      const _Float16 sh = (_Float16)fminf(a / 7.0f, 65504.0f);
      const float sf = (float)sh;
      const float rcp = 1.0f / sf;
      const float hs = 0.5f * sf;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float q0 = rintf(xh[i] * rcp);
        // x - q0 * s is exact whenever it is near s / 2 (see the oracle's argument),
        // so this decides the exact quotient's rounding, ties to even.
        const float e = fmaf(-q0, sf, xh[i]);
        const float ae = fabsf(e);
        const bool odd = (((int)q0) & 1) != 0;
        const bool away = (ae > hs) || (ae == hs && odd);
        float q = away ? q0 + copysignf(1.0f, e) : q0;
        q = fminf(fmaxf(q, -7.0f), 7.0f);
        const int qi = (sf == 0.0f) ? 0 : (int)q;
        nib[i] = (uint32_t)((qi < 0 ? 8 : 0) | (qi < 0 ? -qi : qi));
      }
      if (row_ok && sub == 0)
        reinterpret_cast<uint16_t*>(sXv)[(int64_t)c * M + row] = __builtin_bit_cast(uint16_t, sh);
    } else {
      // MXFP4: e = smallest exponent with 6 * 2^e >= a (clamped to [-127, 127]);
      // codes = E2M1 round-half-even of x * 2^-e (hardware convert, scale 1).
      const uint32_t ab = __float_as_uint(a);
      const int E = (int)((ab >> 23) & 0xFF);
      int e;
      if (a == 0.0f) e = 0;
      else if (E == 0) e = -127;
      else e = (E - 127) - 2 + (((ab & 0x7FFFFFu) > 0x400000u) ? 1 : 0);
      e = e < -127 ? -127 : (e > 127 ? 127 : e);
      const float inv2e = __uint_as_float((uint32_t)(127 - e) << 23);
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        uint32_t p = 0;
        p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, xh[i] * inv2e, xh[i + 1] * inv2e, 1.0f, 0);
        nib[i] = p & 0xF;
        nib[i + 1] = (p >> 4) & 0xF;
      }
      if (row_ok && (sub & 1) == 0)
        reinterpret_cast<uint8_t*>(sXv)[(int64_t)(2 * c + (sub >> 1)) * M + row] = (uint8_t)(e + 127);
    }
    if (row_ok) {
      uint32_t w0 = 0, w1 = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        w0 |= (nib[2 * j] | (nib[2 * j + 1] << 4)) << (8 * j);
        w1 |= (nib[8 + 2 * j] | (nib[8 + 2 * j + 1] << 4)) << (8 * j);
      }
      *reinterpret_cast<uint2*>(qX + row * (K >> 1) + (k0 >> 1)) = make_uint2(w0, w1);
    }

    if constexpr (NT > 0) {
      const v8bf a0 = __builtin_bit_cast(v8bf, xa);
      const v8bf a1 = __builtin_bit_cast(v8bf, xb);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int n = t * 16 + r16;
        uint4 h0 = make_uint4(0, 0, 0, 0), h1 = h0, l0 = h0, l1 = h0;
        if (n < rank) {
          const uint4* ph = reinterpret_cast<const uint4*>(Ldh + (int64_t)n * K + k0);
          const uint4* pl = reinterpret_cast<const uint4*>(Ldl + (int64_t)n * K + k0);
          h0 = ph[0]; h1 = ph[1]; l0 = pl[0]; l1 = pl[1];
        }
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, __builtin_bit_cast(v8bf, h0), acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, __builtin_bit_cast(v8bf, h1), acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, __builtin_bit_cast(v8bf, l0), acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, __builtin_bit_cast(v8bf, l1), acc[t], 0, 0, 0);
      }
    }
  }

  if constexpr (NT > 0) {
    // D layout of the 16x16 MFMA: lane l holds column l & 15, rows 4 * (l >> 4) + i.
    __shared__ float red[4][16][NT * 16];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave][4 * sub + i][t * 16 + r16] = acc[t][i];
    __syncthreads();
    const int64_t m0 = (int64_t)blockIdx.x * 16;
    for (int idx = threadIdx.x; idx < 16 * rank; idx += 256) {
      const int rr = idx / rank, cc = idx - rr * rank;
      if (m0 + rr < M)
        lora_act[(m0 + rr) * rank + cc] = red[0][rr][cc] + red[1][rr][cc] + red[2][rr][cc] + red[3][rr][cc];
    }
  }
}

template <int FMT>
static hipError_t launch_k1_fmt(const KernelLayer& L, int64_t M, const uint16_t* X, int64_t ldx,
                                uint8_t* qX, void* sX, float* lora_act, hipStream_t st) {
  const dim3 grid((unsigned)((M + 15) / 16)), block(256);
  const int nt = (L.rank + 15) / 16;
#define K1_CASE(NTV)                                                                          \
  case NTV:                                                                                   \
    hipLaunchKernelGGL((k1_quant_lora_down<FMT, NTV>), grid, block, 0, st, X, ldx, M, L.K,    \
                       L.inv_s, L.Ld_hi, L.Ld_lo, L.rank, qX, sX, lora_act);                  \
    break;
  switch (nt) {
    K1_CASE(0) K1_CASE(1) K1_CASE(2) K1_CASE(3) K1_CASE(4)
    K1_CASE(5) K1_CASE(6) K1_CASE(7) K1_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef K1_CASE
  return hipGetLastError();
}

hipError_t launch_k1(const KernelLayer& L, int64_t M, const uint16_t* X, int64_t ldx, uint8_t* qX,
                     void* sX, float* lora_act, hipStream_t st) {
  if (L.fmt == 0) return launch_k1_fmt<0>(L, M, X, ldx, qX, sX, lora_act, st);
  return launch_k1_fmt<1>(L, M, X, ldx, qX, sX, lora_act, st);
}

}  // namespace svdq
