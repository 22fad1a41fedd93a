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
// Work split: a block of 8 waves owns 16 consecutive tokens.  The K dimension is cut
// into 64-wide chunks; wave w takes chunks w, w+8, ..., with the next chunk's X, inv_s
// and L1 loads issued before the current chunk is processed.  Inside a chunk, lane l holds
// token (l & 15) and the 16 consecutive channels 16 * (l >> 4) .. +15.  One INT4 group
// (64) is therefore spread over the 4 lanes l, l^16, l^32, l^48; one FP4 group (32)
// over lanes l, l^16.  X is loaded row-contiguously instead (each 16-byte load covers 8
// whole 128-byte lines of 8 tokens) and regrouped through a small per-wave LDS tile:
// loads whose 4-lane groups straddle 4 lines were measured markedly slower.
//
// Down projection: X_hat L1 with L1 in bf16, prepared in fragment order: for one chunk
// and one tile of 16 rank columns, the 32 bytes a lane needs (16 channels of one rank
// column) are contiguous, so each 16-byte load reads whole 128-byte lines (the plain
// [rank][K] rows made every load touch 16 half-used lines, and these loads, repeated by
// every block of 16 tokens, cost more than the pass over X).  The smoothed activations
// exist only in fp32 registers, so each is split into a bf16 pair hi + lo (hi = bf16(x),
// lo = bf16(x - hi): x to ~2^-17) and the pair feeds two v_mfma_f32_16x16x32_bf16
// against the same L1 fragment, which keeps the low-rank branch fp32-accurate with one
// read of L1 per chunk.  Lane l supplies MFMA row l & 15 and k-block l >> 4: the lane's
// first 8 channels go to one MFMA and the next 8 to a second, and the B operand uses
// the same channel order.  Partial sums of the waves are added through LDS at the end,
// in a fixed order.
//
// INT4 rounding: t = x * (1 / s) is within |x / s| * 2^-23 of the quotient x / s, so
// round(t) is the correctly rounded code unless x / s lies within 2^-17 of a half
// integer.  Such lanes are flagged and, if any lane of the wave has one, the chunk takes
// the exact correction (x - q * s is exact near s / 2, and ties go to even).  The MMA
// form then converts t / 8 with the hardware FP6 conversion (round to nearest even on
// the E2M3 subnormal grid, whose step is 1/8): the 6-bit field of code q, value q / 8.
// The converter interleaves two 16-value inputs field by field, so the lanes of
// quarters 2h and 2h+1 of a group (lanes l and l ^ 16) each convert their own 16 codes
// twice, exchange halves with one row swap per word, and keep the even fields of the
// even quarter and the odd fields of the odd quarter: field f of half h holds
// k = 32 h + 16 (f & 1) + (f >> 1), the order kernel 2's weight operand uses.
#include "common.hpp"
#include "kernels.hpp"

namespace svdq {

constexpr int K1_WAVES = 8;

typedef __bf16 bf2 __attribute__((ext_vector_type(2)));

// fp32 pair -> bf16 pair bits, round to nearest even (element a in the low half)
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  const bf2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Rank tiles 0-2 fit in 128 VGPRs, so two 8-wave blocks share a CU.
// QUANT = false: the down projection alone (lora_act only), the unfused baseline's
// separate low-rank pass over X; qX and sX are not touched.
template <int FMT, int NT, bool MMA, bool QUANT = true>
__global__ __launch_bounds__(64 * K1_WAVES) __attribute__((amdgpu_waves_per_eu(NT <= 2 ? 4 : 2))) void
k1_quant_lora_down(const uint16_t* __restrict__ X, int64_t ldx, int64_t M, int64_t K,
                   const float* __restrict__ inv_s, const uint16_t* __restrict__ L1f, int rank,
                   uint8_t* __restrict__ qX, void* __restrict__ sXv, float* __restrict__ lora_act) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r16 = lane & 15;
  const int sub = lane >> 4;
  const int64_t m0 = (int64_t)blockIdx.x * 16;
  const int64_t row = m0 + r16;
  const bool row_ok = row < M;
  const int nchunks = (int)(K >> 6);
  // rows past M read as zeros through the range check
  const int64_t nrows = M - m0 < 16 ? M - m0 : 16;
  const __amdgpu_buffer_rsrc_t rX = make_rsrc(X + m0 * ldx, (uint32_t)(((nrows - 1) * ldx + K) * 2));
  const __amdgpu_buffer_rsrc_t rS = make_rsrc(inv_s, (uint32_t)(K * 4));
  // X loads: lane l takes row 8 i + (l >> 3), 16-byte piece l & 7 of the chunk's 128
  // bytes (load i = 0, 1), so each load reads 8 whole lines; the pieces are regrouped
  // to the lane's (row l & 15, 32 bytes at 32 (l >> 4)) through a per-wave LDS tile.
  const uint32_t xoff = (uint32_t)((lane >> 3) * ldx + (lane & 7) * 8) * 2;
  const uint32_t xstep8 = (uint32_t)(8 * ldx * 2);
  __shared__ uint4 xs[K1_WAVES][16][9];
  const __amdgpu_buffer_rsrc_t rL = make_rsrc(L1f, (uint32_t)(NT * 16 * K * 2));

  v4f acc[NT > 0 ? NT : 1];
#pragma unroll
  for (int t = 0; t < (NT > 0 ? NT : 1); ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};

  // One chunk ahead: X, the lane's own inv_s element (channel sub * 16 + r16: the 16
  // lanes of a row hold the row's 16 channels, broadcast to the row where they are
  // used) and the L1 fragments (rows past the rank are zero in the prepared layout).
  uint4 xa, xb, LAn[NT > 0 ? NT : 1], LBn[NT > 0 ? NT : 1];
  uint32_t sv;
  auto fetch = [&](int c) {
    const uint32_t kx = xoff + (uint32_t)c * 128;
    xa = buf_load16(rX, kx);
    xb = buf_load16(rX, kx + xstep8);
    sv = buf_load4(rS, (uint32_t)(c * 64 + sub * 16 + r16) * 4);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      // fragment order: lane l's 32 bytes of chunk c, rank tile t, contiguous
      const uint32_t o = (uint32_t)(((c * NT + t) * 64 + lane) * 32);
      LAn[t] = buf_load16(rL, o);
      LBn[t] = buf_load16(rL, o + 16);
    }
  };
  if (wave < nchunks) fetch(wave);

  for (int c = wave; c < nchunks; c += K1_WAVES) {
    const int64_t k0 = (int64_t)c * 64 + sub * 16;
    xs[wave][lane >> 3][lane & 7] = xa;
    xs[wave][8 + (lane >> 3)][lane & 7] = xb;
    const uint4 ya = xs[wave][r16][2 * sub], yb = xs[wave][r16][2 * sub + 1];
    const uint32_t xw[8] = {ya.x, ya.y, ya.z, ya.w, yb.x, yb.y, yb.z, yb.w};
    const int s_own = (int)sv;
    uint4 LA[NT > 0 ? NT : 1], LB[NT > 0 ? NT : 1];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      LA[t] = LAn[t];
      LB[t] = LBn[t];
    }
    if (c + K1_WAVES < nchunks) fetch(c + K1_WAVES);

    // x * inv_s, inv_s of channel i from lane i of the row (DPP row_newbcast:i)
#define K1_BC(i) __int_as_float(__builtin_amdgcn_update_dpp(0, s_own, 0x150 + (i), 0xF, 0xF, false))
    float xh[16];
    xh[0] = bf16_lo_to_f32(xw[0]) * K1_BC(0);
    xh[1] = bf16_hi_to_f32(xw[0]) * K1_BC(1);
    xh[2] = bf16_lo_to_f32(xw[1]) * K1_BC(2);
    xh[3] = bf16_hi_to_f32(xw[1]) * K1_BC(3);
    xh[4] = bf16_lo_to_f32(xw[2]) * K1_BC(4);
    xh[5] = bf16_hi_to_f32(xw[2]) * K1_BC(5);
    xh[6] = bf16_lo_to_f32(xw[3]) * K1_BC(6);
    xh[7] = bf16_hi_to_f32(xw[3]) * K1_BC(7);
    xh[8] = bf16_lo_to_f32(xw[4]) * K1_BC(8);
    xh[9] = bf16_hi_to_f32(xw[4]) * K1_BC(9);
    xh[10] = bf16_lo_to_f32(xw[5]) * K1_BC(10);
    xh[11] = bf16_hi_to_f32(xw[5]) * K1_BC(11);
    xh[12] = bf16_lo_to_f32(xw[6]) * K1_BC(12);
    xh[13] = bf16_hi_to_f32(xw[6]) * K1_BC(13);
    xh[14] = bf16_lo_to_f32(xw[7]) * K1_BC(14);
    xh[15] = bf16_hi_to_f32(xw[7]) * K1_BC(15);
#undef K1_BC
    if constexpr (QUANT) {
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) a = fmaxf(a, fabsf(xh[i]));
    a = wave_max_xor(a, 16);

    if constexpr (FMT == 0) {
      // INT4: s = fp16(fp32(a / 7)), saturating; q = round-half-even(x / s) exactly
      a = wave_max_xor(a, 32);
      const _Float16 sh = (_Float16)fminf(a / 7.0f, 65504.0f);
      const float sf = (float)sh;
      const float rcp = sf > 0.0f ? 1.0f / sf : 0.0f;  // s = 0: every x is 0, every code 0
      float t[16];
      float dev = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        t[i] = xh[i] * rcp;
        dev = fmaxf(dev, fabsf(t[i] - rintf(t[i])));
      }
      if (__builtin_amdgcn_ballot_w64(dev > 0.49999237f) != 0) {  // 0.5 - 2^-17
        const float hs = 0.5f * sf;
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
      // MMA form: a group half's 192-bit operand (six words), built by the lane pair of
      // quarters 2h, 2h+1 together (every lane takes part in the row swap, valid row or
      // not).  The clamp to +-7 only acts for subnormal fp16 scales; code 0 may carry
      // either sign bit.
      uint32_t fw[3] = {0u, 0u, 0u};
      if constexpr (MMA) {
        v16f tc;
#pragma unroll
        for (int i = 0; i < 16; ++i) tc[i] = __builtin_amdgcn_fmed3f(t[i], -7.0f, 7.0f);
        const v6i f6 = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(tc, tc, 8.0f);
        // bits of the even fields (field 2i at bit 12 i) in words d and d + 3
        constexpr uint32_t EV[3] = {0x3F03F03Fu, 0xF03F03F0u, 0x03F03F03u};
#pragma unroll
        for (int d = 0; d < 3; ++d) {
          // even rows (quarters 0, 2) receive the odd row's word d, odd rows the even
          // row's word d + 3
          const auto r = __builtin_amdgcn_permlane16_swap((uint32_t)f6[d], (uint32_t)f6[d + 3], false, false);
          fw[d] = (r[0] & EV[d]) | (r[1] & ~EV[d]);
        }
      }
      if (row_ok) {
        if constexpr (MMA) {
          // [M][K/64][64] bytes per token and group: quarter q stores 16 bytes at 16 q,
          // words 0-2 (quarter 2h) or 3-5 (quarter 2h+1) of half h, then a zero word
          *reinterpret_cast<uint4*>(qX + row * K + k0) = make_uint4(fw[0], fw[1], fw[2], 0u);
        } else {
          uint32_t w0 = 0, w1 = 0;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float qc = __builtin_amdgcn_fmed3f(rintf(t[i]), -7.0f, 7.0f);
            const uint32_t nib = (uint32_t)fabsf(qc) | (qc < 0.0f ? 8u : 0u);
            if (i < 8) w0 |= nib << (4 * i);
            else w1 |= nib << (4 * (i - 8));
          }
          *reinterpret_cast<uint2*>(qX + row * (K >> 1) + (k0 >> 1)) = make_uint2(w0, w1);
        }
        if (sub == 0) {
          if constexpr (MMA) {  // fp16 bits, rows padded to 4
            const int64_t Mp = (M + 3) & ~int64_t(3);
            reinterpret_cast<uint16_t*>(sXv)[(int64_t)c * Mp + row] = __builtin_bit_cast(uint16_t, sh);
          } else {
            reinterpret_cast<uint16_t*>(sXv)[(int64_t)c * M + row] = __builtin_bit_cast(uint16_t, sh);
          }
        }
      }
    } else {
      // MXFP4: e = smallest exponent with 6 * 2^e >= a (clamped to [-127, 127]);
      // codes = E2M1 round-half-even of x * 2^-e (hardware convert, scale 1), each
      // pair converted straight into its byte of the packed word.
      const uint32_t ab = __float_as_uint(a);
      const int E = (int)((ab >> 23) & 0xFF);
      int e;
      if (a == 0.0f) e = 0;
      else if (E == 0) e = -127;
      else e = (E - 127) - 2 + (((ab & 0x7FFFFFu) > 0x400000u) ? 1 : 0);
      e = e < -127 ? -127 : (e > 127 ? 127 : e);
      const float inv2e = __uint_as_float((uint32_t)(127 - e) << 23);
      float y[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) y[i] = xh[i] * inv2e;
      uint32_t w0 = 0, w1 = 0;  // the byte index operand must be a literal
      w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, y[0], y[1], 1.0f, 0);
      w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, y[2], y[3], 1.0f, 1);
      w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, y[4], y[5], 1.0f, 2);
      w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, y[6], y[7], 1.0f, 3);
      w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, y[8], y[9], 1.0f, 0);
      w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, y[10], y[11], 1.0f, 1);
      w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, y[12], y[13], 1.0f, 2);
      w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, y[14], y[15], 1.0f, 3);
      if (row_ok) {
        const int64_t b = k0 >> 1;  // byte of the token's code row
        // MMA form: token pairs, the 64-byte segments (128 K values, one kernel-2 stage)
        // of tokens 2j and 2j+1 share a 128-byte line
        uint8_t* dst = MMA ? qX + (row >> 1) * K + (b >> 6) * 128 + (row & 1) * 64 + (b & 63) : qX + row * (K >> 1) + b;
        *reinterpret_cast<uint2*>(dst) = make_uint2(w0, w1);
        if ((sub & 1) == 0) {
          const int64_t ld = MMA ? (M + 3) & ~int64_t(3) : M;  // MMA form: rows padded to 4
          reinterpret_cast<uint8_t*>(sXv)[(int64_t)(2 * c + (sub >> 1)) * ld + row] = (uint8_t)(e + 127);
        }
      }
    }
    }  // QUANT

    if constexpr (NT > 0) {
      // x = hi + lo as bf16 pairs, channels 0-7 of the lane in a*0, 8-15 in a*1
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

  if constexpr (NT > 0) {
    // D layout of the 16x16 MFMA: lane l holds column l & 15, rows 4 * (l >> 4) + i.
    __shared__ float red[K1_WAVES][16][NT * 16];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave][4 * sub + i][t * 16 + r16] = acc[t][i];
    __syncthreads();
    // all NT * 16 columns are written; those past the rank are zero (their L1 rows are
    // as zeros)
    constexpr int R16 = NT * 16;
    for (int idx = threadIdx.x; idx < 16 * R16; idx += 64 * K1_WAVES) {
      const int rr = idx / R16, cc = idx - rr * R16;
      if (m0 + rr < M) {
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < K1_WAVES; ++w) v += red[w][rr][cc];
        if constexpr (MMA) {
          // the bf16 pair kernel 2's up-projection MFMA consumes, v = hi + lo to ~2^-17
          // relative, in its fragment order: 32-row blocks, k steps of 16, hi then lo
          // (512 elements apart), the 64 lanes' 8 values (lane m % 32 + 32 (k / 8 % 2))
          const uint32_t hb = f32_to_bf16_rne(v);
          const uint32_t lb = f32_to_bf16_rne(v - __uint_as_float(hb << 16));
          const int64_t m = m0 + rr;
          uint16_t* la = reinterpret_cast<uint16_t*>(lora_act) +
                         (((((m >> 5) * NT + (cc >> 4)) * 2) * 64 + (m & 31) + 32 * ((cc >> 3) & 1)) << 3) + (cc & 7);
          la[0] = (uint16_t)hb;
          la[512] = (uint16_t)lb;
        } else {
          lora_act[(m0 + rr) * R16 + cc] = v;
        }
      }
    }
  }
}

template <int FMT, bool MMA>
static hipError_t launch_k1_fmt(const KernelLayer& L, int64_t M, const uint16_t* X, int64_t ldx,
                                uint8_t* qX, void* sX, void* lora_act, hipStream_t st) {
  const dim3 grid((unsigned)((M + 15) / 16));
  const int nt = (L.rank + 15) / 16;
#define K1_CASE(NTV)                                                                            \
  case NTV:                                                                                     \
    hipLaunchKernelGGL((k1_quant_lora_down<FMT, NTV, MMA>), grid, dim3(64 * K1_WAVES), 0, st, X, ldx, M, L.K, \
                       L.inv_s, L.L1f, L.rank, qX, sX, static_cast<float*>(lora_act));                    \
    break;
  switch (nt) {
    K1_CASE(0) K1_CASE(1) K1_CASE(2) K1_CASE(3) K1_CASE(4)
    K1_CASE(5) K1_CASE(6) K1_CASE(7) K1_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef K1_CASE
  return hipGetLastError();
}

hipError_t launch_k1_down(const KernelLayer& L, int64_t M, const uint16_t* X, int64_t ldx, void* lora_act,
                          hipStream_t st) {
  const dim3 grid((unsigned)((M + 15) / 16));
#define K1D_CASE(NTV)                                                                                          \
  case NTV:                                                                                                    \
    hipLaunchKernelGGL((k1_quant_lora_down<0, NTV, true, false>), grid, dim3(64 * K1_WAVES), 0, st, X, ldx, M, L.K, L.inv_s, \
                       L.L1f, L.rank, (uint8_t*)nullptr, (void*)nullptr, static_cast<float*>(lora_act));       \
    break;
  switch ((L.rank + 15) / 16) {
    K1D_CASE(1) K1D_CASE(2) K1D_CASE(3) K1D_CASE(4) K1D_CASE(5) K1D_CASE(6) K1D_CASE(7) K1D_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef K1D_CASE
  return hipGetLastError();
}

hipError_t launch_k1(const KernelLayer& L, int64_t M, const uint16_t* X, int64_t ldx, uint8_t* qX,
                     void* sX, void* lora_act, bool mma, hipStream_t st) {
  if (L.fmt == 0)
    return mma ? launch_k1_fmt<0, true>(L, M, X, ldx, qX, sX, lora_act, st)
               : launch_k1_fmt<0, false>(L, M, X, ldx, qX, sX, lora_act, st);
  return mma ? launch_k1_fmt<1, true>(L, M, X, ldx, qX, sX, lora_act, st)
             : launch_k1_fmt<1, false>(L, M, X, ldx, qX, sX, lora_act, st);
}

}  // namespace svdq
