// Kernel 2: W4A4 GEMM on the 4-bit codes, per-group rescale by s_X s_W, low-rank up
// projection (X_hat L1) L2 added in the epilogue.
//
// Method: the scaled low-bit product XW ~ s_X s_W Q_X Q_W (jeonghoonpark.com "SVDQuant"
// review, section 3), taken per K-group, plus the 16-bit low-rank branch of the
// decomposition equation (review, section 4.2), with the up projection fused into the
// 4-bit GEMM (review, section 4.3, Figure 6(b)).
//
// Matrix cores: v_mfma_scale_f32_32x32x64_f8f6f4.
//  * MXFP4: the E2M1 codes are the operands as stored and the E8M0 group scales are
//    the hardware block scales; the MFMA accumulates the exact scaled products.
//  * INT4: a sign-magnitude code q becomes the FP8 E4M3 byte (sign, exponent 0,
//    mantissa |q|), whose value is q * 2^-9 (a subnormal; exact).  Each fp16 group
//    scale s = m * 2^e (m in [1,2)) is split: 2^(e+9) goes to the MFMA's E8M0 block
//    scale, so one MFMA yields the exact group sum times 2^(eX+eW) in fp32, and the
//    epilogue adds it times the fp16 product mX*mW (v_pk_mul_f16 + v_fma_mix_f32).
//    With per-group scales on both sides this per-element rescale is the VALU cost
//    that bounds the INT4 path; moving the powers of two into the MFMA halves it.
//
// Tiling: a 512-thread block (8 waves) owns a 256 x 256 output tile; wave w owns rows
// 128*(w/4) .. +127 and columns 64*(w%4) .. +63, i.e. 4 x 2 MFMA tiles of 32 x 32.  Per
// 64-wide K step the block stages both operand panels through LDS (double buffered,
// rows padded to avoid bank conflicts); the codes are expanded once per block there.
//
// 32x32x64 operand layout (measured): lane l supplies row/column l & 31; for FP4 it
// holds the 32 consecutive K values 32*(l>>5).. with the block scale of that half; for
// FP8 the k order inside the lane differs but a group's single scale covers both
// halves, so A and B only need the same byte order.  Output: lane l holds column
// l & 31, rows 8*(a>>2) + 4*(l>>5) + (a&3) for accumulator a = 0..15.
#include "common.hpp"
#include "kernels.hpp"

namespace svdq {

namespace {

constexpr int BM = 256, BN = 256, NWAVES = 8, NTHREADS = 512;
constexpr int WM = 128, WN = 64;  // wave tile
constexpr int TI = WM / 32, TJ = WN / 32;

template <int FMT>
struct Smem {
  // operand row pitch in bytes: INT4 expands 32 code bytes to 64 FP8 bytes
  static constexpr int kRow = FMT == 0 ? 64 : 32;
  static constexpr int kPitch = kRow + 16;
  uint8_t A[2][BM * kPitch];
  uint8_t B[2][BN * kPitch];
  _Float16 mX[2][BM];
  _Float16 mW[2][BN];
  uint32_t eX[2][BM];  // MXFP4: two E8M0 bytes (groups 2s, 2s+1); INT4: one byte
  uint32_t eW[2][BN];
};

// fp16 scale -> (fp16 mantissa in [1,2) or 0, E8M0 byte for 2^(e+9))
__device__ __forceinline__ void split_scale(uint16_t bits, _Float16& m, uint32_t& ebyte) {
  const float f = (float)__builtin_bit_cast(_Float16, bits);
  if (f == 0.0f) {
    m = (_Float16)0.0f;
    ebyte = 127;
    return;
  }
  const uint32_t u = __float_as_uint(f);
  const int e = (int)((u >> 23) & 0xFF) - 127;
  m = (_Float16)__uint_as_float((u & 0x807FFFFFu) | (127u << 23));
  ebyte = (uint32_t)(e + 9 + 127);
}

template <int FMT, bool DEBUG>
__global__ __launch_bounds__(NTHREADS) void k2_gemm(
    const uint8_t* __restrict__ qX, const void* __restrict__ sXv, int64_t M,
    const uint8_t* __restrict__ qW, const void* __restrict__ sWv, int64_t N, int64_t K,
    const float* __restrict__ lora_act, const uint16_t* __restrict__ L2, int rank,
    void* __restrict__ Y, int64_t ldy, int ydtype,
    int64_t mbase, int64_t nbase, int64_t mlim, int64_t nlim, int32_t* __restrict__ dbg) {
  using S = Smem<FMT>;
  __shared__ S sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int kh = lane >> 5;
  const int wm = (wave >> 2) * WM;
  const int wn = (wave & 3) * WN;
  const int64_t m0 = mbase + (int64_t)blockIdx.y * BM;
  const int64_t n0 = nbase + (int64_t)blockIdx.x * BN;
  const int64_t Kb = K >> 1;            // bytes per code row
  const int nsteps = (int)(K >> 6);     // 64-wide K steps

  // ---- global -> register staging (one 16-byte piece of A and of B per thread) ----
  const int ldrow = tid >> 1, ldhalf = tid & 1;
  const int64_t arow = m0 + ldrow, brow = n0 + ldrow;
  const bool a_ok = arow < mlim, b_ok = brow < nlim;
  const uint8_t* pa = qX + arow * Kb + ldhalf * 16;
  const uint8_t* pb = qW + brow * Kb + ldhalf * 16;
  uint4 ra, rb;
  uint32_t rs;  // scale bits for row/col tid (tid < 256: X row, else W column)
  auto gload = [&](int s) {
    ra = a_ok ? *reinterpret_cast<const uint4*>(pa + (int64_t)s * 32) : make_uint4(0, 0, 0, 0);
    rb = b_ok ? *reinterpret_cast<const uint4*>(pb + (int64_t)s * 32) : make_uint4(0, 0, 0, 0);
    if (DEBUG) {
      rs = 0x3C00u;  // unit scale; the debug epilogue forces its own scale bytes
    } else if (tid < BM) {
      const int64_t r = m0 + tid;
      if (FMT == 0) rs = r < mlim ? reinterpret_cast<const uint16_t*>(sXv)[(int64_t)s * M + r] : 0;
      else rs = r < mlim ? (uint32_t)reinterpret_cast<const uint8_t*>(sXv)[(int64_t)(2 * s) * M + r] |
                               ((uint32_t)reinterpret_cast<const uint8_t*>(sXv)[(int64_t)(2 * s + 1) * M + r] << 8)
                         : 0x7F7Fu;
    } else {
      const int64_t c = n0 + tid - BM;
      if (FMT == 0) rs = c < nlim ? reinterpret_cast<const uint16_t*>(sWv)[(int64_t)s * N + c] : 0;
      else rs = c < nlim ? (uint32_t)reinterpret_cast<const uint8_t*>(sWv)[(int64_t)(2 * s) * N + c] |
                               ((uint32_t)reinterpret_cast<const uint8_t*>(sWv)[(int64_t)(2 * s + 1) * N + c] << 8)
                         : 0x7F7Fu;
    }
  };
  auto sstore = [&](int buf) {
    if (FMT == 0) {
      uint32_t a8[8], b8[8];
      const uint32_t aw[4] = {ra.x, ra.y, ra.z, ra.w}, bw[4] = {rb.x, rb.y, rb.z, rb.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        nib8_to_fp8(aw[i], a8[2 * i], a8[2 * i + 1]);
        nib8_to_fp8(bw[i], b8[2 * i], b8[2 * i + 1]);
      }
      uint4* da = reinterpret_cast<uint4*>(&sm.A[buf][ldrow * S::kPitch + ldhalf * 32]);
      uint4* db = reinterpret_cast<uint4*>(&sm.B[buf][ldrow * S::kPitch + ldhalf * 32]);
      da[0] = make_uint4(a8[0], a8[1], a8[2], a8[3]);
      da[1] = make_uint4(a8[4], a8[5], a8[6], a8[7]);
      db[0] = make_uint4(b8[0], b8[1], b8[2], b8[3]);
      db[1] = make_uint4(b8[4], b8[5], b8[6], b8[7]);
      _Float16 m;
      uint32_t eb;
      split_scale((uint16_t)rs, m, eb);
      if (DEBUG) {
        m = (_Float16)1.0f;
        eb = 127 + 9;
      }
      if (tid < BM) { sm.mX[buf][tid] = m; sm.eX[buf][tid] = eb; }
      else { sm.mW[buf][tid - BM] = m; sm.eW[buf][tid - BM] = eb; }
    } else {
      *reinterpret_cast<uint4*>(&sm.A[buf][ldrow * S::kPitch + ldhalf * 16]) = ra;
      *reinterpret_cast<uint4*>(&sm.B[buf][ldrow * S::kPitch + ldhalf * 16]) = rb;
      if (tid < BM) sm.eX[buf][tid] = rs;
      else sm.eW[buf][tid - BM] = rs;
    }
  };

  v16f acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = v16f{};

  gload(0);
  sstore(0);
  __syncthreads();

  for (int s = 0; s < nsteps; ++s) {
    const int buf = s & 1;
    if (s + 1 < nsteps) gload(s + 1);

    // B fragments and column scales of this wave
    v8i bf[TJ];
    uint32_t sb[TJ];
    _Float16 mw[TJ];
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int col = wn + j * 32 + l32;
      if (FMT == 0) {
        const uint4* p = reinterpret_cast<const uint4*>(&sm.B[buf][col * S::kPitch + kh * 32]);
        const uint4 x0 = p[0], x1 = p[1];
        bf[j] = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
        sb[j] = sm.eW[buf][col];
        mw[j] = sm.mW[buf][col];
      } else {
        const uint4 x0 = *reinterpret_cast<const uint4*>(&sm.B[buf][col * S::kPitch + kh * 16]);
        bf[j] = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, 0, 0, 0, 0};
        sb[j] = (sm.eW[buf][col] >> (8 * kh)) & 0xFF;
      }
    }
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const int row = wm + i * 32 + l32;
      v8i af;
      uint32_t sa;
      if (FMT == 0) {
        const uint4* p = reinterpret_cast<const uint4*>(&sm.A[buf][row * S::kPitch + kh * 32]);
        const uint4 x0 = p[0], x1 = p[1];
        af = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
        sa = sm.eX[buf][row];
      } else {
        const uint4 x0 = *reinterpret_cast<const uint4*>(&sm.A[buf][row * S::kPitch + kh * 16]);
        af = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, 0, 0, 0, 0};
        sa = (sm.eX[buf][row] >> (8 * kh)) & 0xFF;
      }
      if (FMT == 0) {
        // mantissas of the 16 accumulator rows: rows 8*(a>>2) + 4*kh + (a&3)
        h2 mx[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int rb0 = wm + i * 32 + 8 * q + 4 * kh;
          const uint2 w = *reinterpret_cast<const uint2*>(&sm.mX[buf][rb0]);
          mx[2 * q] = __builtin_bit_cast(h2, w.x);
          mx[2 * q + 1] = __builtin_bit_cast(h2, w.y);
        }
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          const v16f p = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af, bf[j], v16f{}, 0, 0, 0,
                                                                        (int)sa, 0, (int)sb[j]);
          if (DEBUG) {
#pragma unroll
            for (int a = 0; a < 16; ++a) {
              const int64_t r = m0 + wm + i * 32 + 8 * (a >> 2) + 4 * kh + (a & 3);
              const int64_t c = n0 + wn + j * 32 + l32;
              if (r < mlim && c < nlim)
                dbg[((int64_t)s * (mlim - mbase) + (r - mbase)) * (nlim - nbase) + (c - nbase)] = (int32_t)p[a];
            }
          } else {
            const h2 mw2 = h2{mw[j], mw[j]};
#pragma unroll
            for (int q = 0; q < 8; ++q) {
              const h2 sc = mx[q] * mw2;
              acc[i][j][2 * q] = fmaf(p[2 * q], (float)sc.x, acc[i][j][2 * q]);
              acc[i][j][2 * q + 1] = fmaf(p[2 * q + 1], (float)sc.y, acc[i][j][2 * q + 1]);
            }
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < TJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af, bf[j], acc[i][j], 4, 4, 0,
                                                                     (int)sa, 0, (int)sb[j]);
      }
    }
    if (s + 1 < nsteps) sstore(buf ^ 1);
    __syncthreads();
  }
  if (DEBUG) return;

  // ---- low-rank up projection: acc += lora_act[rows, :] L2[:, cols] -------------------
  // v_mfma_f32_32x32x16_bf16 with a bf16 hi/lo split of lora_act (L2 is bf16 already).
  if (rank > 0) {
    for (int k0 = 0; k0 < rank; k0 += 16) {
      v8bf bl[TJ];
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int64_t c = n0 + wn + j * 32 + l32;
        uint16_t t[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int k = k0 + 8 * kh + u;
          t[u] = (k < rank && c < nlim) ? L2[(int64_t)k * N + c] : (uint16_t)0;
        }
        bl[j] = __builtin_bit_cast(v8bf, t);
      }
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        const int64_t r = m0 + wm + i * 32 + l32;
        uint16_t hi[8], lo[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int k = k0 + 8 * kh + u;
          const float v = (k < rank && r < mlim) ? lora_act[r * rank + k] : 0.0f;
          const uint32_t hb = f32_to_bf16_rne(v);
          hi[u] = (uint16_t)hb;
          lo[u] = (uint16_t)f32_to_bf16_rne(v - __uint_as_float(hb << 16));
        }
        const v8bf ah = __builtin_bit_cast(v8bf, hi), al = __builtin_bit_cast(v8bf, lo);
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bl[j], acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bl[j], acc[i][j], 0, 0, 0);
        }
      }
    }
  }

  // ---- store -------------------------------------------------------------------------
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int64_t c = n0 + wn + j * 32 + l32;
      if (c >= nlim) continue;
#pragma unroll
      for (int a = 0; a < 16; ++a) {
        const int64_t r = m0 + wm + i * 32 + 8 * (a >> 2) + 4 * kh + (a & 3);
        if (r < mlim) {
          if (ydtype == 0) reinterpret_cast<float*>(Y)[r * ldy + c] = acc[i][j][a];
          else reinterpret_cast<uint16_t*>(Y)[r * ldy + c] = (uint16_t)f32_to_bf16_rne(acc[i][j][a]);
        }
      }
    }
}

}  // namespace

hipError_t launch_k2(const KernelLayer& L, int64_t M, const uint8_t* qX, const void* sX,
                     const float* lora_act, void* Y, int64_t ldy, int ydtype, hipStream_t st) {
  const dim3 grid((unsigned)((L.N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM)), block(NTHREADS);
  if (L.fmt == 0)
    hipLaunchKernelGGL((k2_gemm<0, false>), grid, block, 0, st, qX, sX, M, L.qW, L.sW, L.N, L.K,
                       lora_act, L.L2, L.rank, Y, ldy, ydtype, (int64_t)0, (int64_t)0, M, L.N,
                       (int32_t*)nullptr);
  else
    hipLaunchKernelGGL((k2_gemm<1, false>), grid, block, 0, st, qX, sX, M, L.qW, L.sW, L.N, L.K,
                       lora_act, L.L2, L.rank, Y, ldy, ydtype, (int64_t)0, (int64_t)0, M, L.N,
                       (int32_t*)nullptr);
  return hipGetLastError();
}

hipError_t launch_k2_debug(const KernelLayer& L, int64_t M, const uint8_t* qX, int64_t m0,
                           int64_t n0, int64_t mt, int64_t nt, int32_t* out, hipStream_t st) {
  const dim3 grid((unsigned)((nt + BN - 1) / BN), (unsigned)((mt + BM - 1) / BM)), block(NTHREADS);
  hipLaunchKernelGGL((k2_gemm<0, true>), grid, block, 0, st, qX, (const void*)nullptr, M, L.qW,
                     (const void*)nullptr, L.N, L.K, (const float*)nullptr, (const uint16_t*)nullptr,
                     0, (void*)nullptr, (int64_t)0, 0, m0, n0, m0 + mt, n0 + nt, out);
  return hipGetLastError();
}

}  // namespace svdq
