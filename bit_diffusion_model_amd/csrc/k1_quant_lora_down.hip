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
// and L1 loads issued before the current chunk is processed.  (The chunks of a block can
// also be cut into a few contiguous ranges, one block each, with the down-projection
// sums of the ranges added by a second small kernel: every block at long K, and at
// short K and rank 0 only the blocks of a last, partly filled round of one block per CU.)  Inside a chunk, lane l holds
// token (l & 15) and the 16 consecutive channels 16 * (l >> 4) .. +15.  One INT4 group
// (64) is therefore spread over the 4 lanes l, l^16, l^32, l^48; one MXFP4 group (32)
// over lanes l, l^16; an NVFP4 group (16) is one lane's 16 values.  X is loaded row-contiguously instead (each 16-byte load covers 8
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
// INT4 rounding: t = x * rcp(s) is within |x / s| * 2^-22 of the quotient x / s, so
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
#include "k1_parts.hpp"
#include "kernels.hpp"

namespace svdq {

constexpr int K1_WAVES = 8;


// Rank tiles 0-2 fit in 128 VGPRs, so two 8-wave blocks share a CU.
// QUANT = false: the down projection alone (lora_act only), the unfused baseline's
// separate low-rank pass over X; qX and sX are not touched.
template <int FMT, int NT, bool MMA, bool QUANT = true>
__global__ __launch_bounds__(64 * K1_WAVES) __attribute__((amdgpu_waves_per_eu(NT <= 2 ? 4 : 2))) void
k1_quant_lora_down(const uint16_t* __restrict__ X, int64_t ldx, int64_t M, int64_t K,
                   const float* __restrict__ inv_s, const uint16_t* __restrict__ L1f, int rank,
                   uint8_t* __restrict__ qX, void* __restrict__ sXv, float* __restrict__ lora_act,
                   float tsx, float r6x, int parts, float* __restrict__ part_out, int full) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r16 = lane & 15;
  const int sub = lane >> 4;
  // Blocks [0, full) each take 16 tokens over all of K; after them, parts > 1 blocks per
  // remaining 16 tokens: block full + t takes tokens 16 (full + t / parts) .. and part
  // t % parts of the chunks, and its down-projection sums go to part_out (rows from token
  // 16 full on), which k1_lora_sum adds up.
  const bool cut = blockIdx.x >= (uint32_t)full;
  const uint32_t tb = blockIdx.x - (uint32_t)full;
  const int np = cut ? parts : 1;
  const int part = cut ? (int)(tb % (uint32_t)parts) : 0;
  const int64_t m0 = cut ? ((int64_t)full + tb / (uint32_t)parts) * 16 : (int64_t)blockIdx.x * 16;
  const int64_t row = m0 + r16;
  const bool row_ok = row < M;
  const int nch = (int)(K >> 6);
  const int cbeg = (int)(((int64_t)part * nch) / np);
  const int nchunks = (int)(((int64_t)(part + 1) * nch) / np);  // end of the block's chunks
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
  // Code and scale stores go through buffer resources as unconditional instructions; a
  // lane with nothing to store (a row past M, a lane that does not own the scale) gives
  // the offset kNoStore, which the range check drops.  (With the stores under branches
  // the compiler's wait counts at the top of the chunk loop no longer included them, so
  // every chunk waited for the previous chunk's write acknowledgements.)  Code offsets
  // are block-local: rows m0 .. (token pairs: pairs m0 / 2 ..; m0 is even).
  const int64_t Mp = (M + 3) & ~int64_t(3);
  const bool pairs = MMA && FMT != 0;
  const __amdgpu_buffer_rsrc_t rQ = make_rsrc(
      qX + (pairs ? (m0 >> 1) * K : m0 * (MMA && FMT == 0 ? K : K >> 1)),
      (uint32_t)(pairs ? ((nrows + 1) >> 1) * K : nrows * (MMA && FMT == 0 ? K : K >> 1)));
  const int64_t s_ld = MMA ? Mp : M;  // scale rows: padded to 4 in the MMA form
  const int64_t s_bytes = FMT == 0 ? (K >> 6) * s_ld * 2 : (FMT == 1 ? (K >> 5) * s_ld : (K >> 4) * s_ld);
  const __amdgpu_buffer_rsrc_t rSc = make_rsrc(sXv, (uint32_t)s_bytes);

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
  if (cbeg + wave < nchunks) fetch(cbeg + wave);

  for (int c = cbeg + wave; c < nchunks; c += K1_WAVES) {
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
    // unconditional (past the end the current chunk again, never used), so the loop has
    // no branches around memory instructions
    fetch(c + K1_WAVES < nchunks ? c + K1_WAVES : c);

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
    if constexpr (FMT != 0) {
#pragma unroll
      for (int i = 0; i < 16; ++i) a = fmaxf(a, fabsf(xh[i]));
      // MXFP4: a 32-group spans lanes l, l ^ 16; NVFP4: the lane's 16 are one group
      if constexpr (FMT == 1) a = wave_max_xor(a, 16);
    }

    if constexpr (FMT == 0) {
      // INT4: s = fp16(fp32(a / 7)), saturating; q = round-half-even(x / s) exactly
      float t[16];
      const _Float16 sh = int4_quantize16(xh, t);
      uint4 mw = make_uint4(0u, 0u, 0u, 0u);
      if constexpr (MMA) mw = int4_mma_words(t, sub);  // every lane takes part in the swaps
      if constexpr (MMA) {
        // [M][K/64][64] bytes per token and group: quarter q stores 16 bytes at 16 q, words
        // 0-3 of half h (quarter 2h) or words 4-5 and two zero words (quarter 2h+1)
        buf_store16(mw, rQ, row_ok ? (uint32_t)(r16 * K + k0) : kNoStore);
      } else {
        uint32_t w0 = 0, w1 = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float qc = __builtin_amdgcn_fmed3f(rintf(t[i]), -7.0f, 7.0f);
          const uint32_t nib = (uint32_t)fabsf(qc) | (qc < 0.0f ? 8u : 0u);
          if (i < 8) w0 |= nib << (4 * i);
          else w1 |= nib << (4 * (i - 8));
        }
        buf_store8(make_uint2(w0, w1), rQ, row_ok ? (uint32_t)(r16 * (K >> 1) + (k0 >> 1)) : kNoStore);
      }
      // fp16 scale bits [K/64][s_ld], from the lanes of quarter 0
      buf_store2(__builtin_bit_cast(uint16_t, sh), rSc,
                 row_ok && sub == 0 ? (uint32_t)(((int64_t)c * s_ld + row) * 2) : kNoStore);
    } else if constexpr (FMT == 2) {
      // NVFP4: s = E4M3(fp32(a * r6)) (hardware conversion: round half to even; the
      // input clamped to 448, the largest finite E4M3), sigma = fp32(s * S_X), codes =
      // E2M1 of fp32(x * fp32(1 / sigma)) (hardware conversion, saturating at 6)
      const float t = fminf(a * r6x, 448.0f);
      const uint32_t sb = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(t, t, 0, false) & 0xFFu;
      const float sigma = __builtin_amdgcn_cvt_f32_fp8((int)sb, 0) * tsx;
      const float rcp = sigma > 0.0f ? 1.0f / sigma : 0.0f;
      float y[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) y[i] = xh[i] * rcp;
      uint32_t w0 = 0, w1 = 0;
      w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, y[0], y[1], 1.0f, 0);
      w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, y[2], y[3], 1.0f, 1);
      w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, y[4], y[5], 1.0f, 2);
      w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, y[6], y[7], 1.0f, 3);
      w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, y[8], y[9], 1.0f, 0);
      w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, y[10], y[11], 1.0f, 1);
      w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, y[12], y[13], 1.0f, 2);
      w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, y[14], y[15], 1.0f, 3);
      if constexpr (MMA) {
        // token pairs; inside the 64-block, codes 16 sub + 0..7 at byte 4 sub and 16 sub +
        // 8..15 at byte 16 + 4 sub (the bf16 matrix core's lane order)
        const uint32_t blk = (uint32_t)((r16 >> 1) * K + (c >> 1) * 128 + (r16 & 1) * 64 + (c & 1) * 32);
        buf_store4(w0, rQ, row_ok ? blk + 4 * sub : kNoStore);
        buf_store4(w1, rQ, row_ok ? blk + 16 + 4 * sub : kNoStore);
        // [K/64][Mp][4]
        buf_store1((uint8_t)sb, rSc, row_ok ? (uint32_t)(((int64_t)c * s_ld + row) * 4 + sub) : kNoStore);
      } else {
        buf_store8(make_uint2(w0, w1), rQ, row_ok ? (uint32_t)(r16 * (K >> 1) + (k0 >> 1)) : kNoStore);
        buf_store1((uint8_t)sb, rSc, row_ok ? (uint32_t)((int64_t)(4 * c + sub) * s_ld + row) : kNoStore);
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
      const int64_t b = k0 >> 1;  // byte of the token's code row
      // MMA form: token pairs, the 64-byte segments (128 K values, one kernel-2 stage) of
      // tokens 2j and 2j+1 share a 128-byte line
      const uint32_t dst = (uint32_t)(MMA ? (r16 >> 1) * K + (b >> 6) * 128 + (r16 & 1) * 64 + (b & 63)
                                          : r16 * (K >> 1) + b);
      buf_store8(make_uint2(w0, w1), rQ, row_ok ? dst : kNoStore);
      // E8M0 bytes [K/32][s_ld], from the lanes of quarters 0 and 2
      buf_store1((uint8_t)(e + 127), rSc,
                 row_ok && (sub & 1) == 0 ? (uint32_t)((int64_t)(2 * c + (sub >> 1)) * s_ld + row) : kNoStore);
    }
    }  // QUANT

    lora_down16<NT>(acc, xh, LA, LB);
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
        if (np > 1) {
          const int64_t mc = (int64_t)full * 16;  // first row of the cut blocks
          part_out[((int64_t)part * (M - mc) + (m0 - mc) + rr) * R16 + cc] = v;
        } else if constexpr (MMA) {
          store_lora_mma(reinterpret_cast<uint16_t*>(lora_act), m0 + rr, cc, NT, v);
        } else {
          lora_act[(m0 + rr) * R16 + cc] = v;
        }
      }
    }
  }
}

// The K-split form's second step, for the rows m0 .. M-1 of the cut blocks:
// lora_act[m][j] = sum over p of part_out[p][m - m0][j], in part order (the result does not
// depend on which block finished first), stored like the unsplit kernel's epilogue.
template <bool MMA>
__global__ __launch_bounds__(256) void k1_lora_sum(const float* __restrict__ part_out, int parts, int64_t m0,
                                                   int64_t M, int R16, float* __restrict__ lora_act) {
  const int64_t total = (M - m0) * R16;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  // all parts' loads issued together (parts <= 8), then added in part order
  float w[8];
#pragma unroll
  for (int p = 0; p < 8; ++p) w[p] = p < parts ? part_out[(int64_t)p * total + idx] : 0.0f;
  float v = w[0];
#pragma unroll
  for (int p = 1; p < 8; ++p)
    if (p < parts) v += w[p];
  const int64_t m = m0 + idx / R16;
  const int j = (int)(idx % R16);
  if constexpr (MMA) store_lora_mma(reinterpret_cast<uint16_t*>(lora_act), m, j, R16 >> 4, v);
  else lora_act[m * R16 + j] = v;
}

template <int FMT, bool MMA>
static hipError_t launch_k1_fmt(const KernelLayer& L, int64_t M, const uint16_t* X, int64_t ldx,
                                uint8_t* qX, void* sX, void* lora_act, int parts, float* part_out, int full,
                                hipStream_t st) {
  const int nt = (L.rank + 15) / 16;
  const int64_t nb = (M + 15) / 16;
  if (parts > 8) return hipErrorInvalidValue;  // k1_lora_sum adds at most 8 ranges
  if (parts < 1 || (nt > 0 && !part_out)) parts = 1;  // rank 0: nothing to add across parts
  if (full < 0) full = 0;
  if (parts == 1 || full >= nb) {
    parts = 1;
    full = (int)nb;
  }
  const dim3 grid((unsigned)(full + (nb - full) * parts));
  // NVFP4 level-2 scale of the activations and fp32(1 / fp32(6 S_X))
  const float tsx = L.tscale_x, r6x = FMT == 2 ? 1.0f / (6.0f * L.tscale_x) : 0.0f;
#define K1_CASE(NTV)                                                                            \
  case NTV:                                                                                     \
    hipLaunchKernelGGL((k1_quant_lora_down<FMT, NTV, MMA>), grid, dim3(64 * K1_WAVES), 0, st, X, ldx, M, L.K, \
                       L.inv_s, L.L1f, L.rank, qX, sX, static_cast<float*>(lora_act), tsx, r6x, parts,    \
                       part_out, full);                                                                    \
    break;
  switch (nt) {
    K1_CASE(0) K1_CASE(1) K1_CASE(2) K1_CASE(3) K1_CASE(4)
    K1_CASE(5) K1_CASE(6) K1_CASE(7) K1_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef K1_CASE
  if (parts > 1 && nt > 0) {
    const int64_t m0 = (int64_t)full * 16, total = (M - m0) * nt * 16;
    hipLaunchKernelGGL((k1_lora_sum<MMA>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, part_out, parts,
                       m0, M, nt * 16, static_cast<float*>(lora_act));
  }
  return hipGetLastError();
}

hipError_t launch_k1_down(const KernelLayer& L, int64_t M, const uint16_t* X, int64_t ldx, void* lora_act,
                          hipStream_t st) {
  const dim3 grid((unsigned)((M + 15) / 16));
#define K1D_CASE(NTV)                                                                                          \
  case NTV:                                                                                                    \
    hipLaunchKernelGGL((k1_quant_lora_down<0, NTV, true, false>), grid, dim3(64 * K1_WAVES), 0, st, X, ldx, M, L.K, L.inv_s, \
                       L.L1f, L.rank, (uint8_t*)nullptr, (void*)nullptr, static_cast<float*>(lora_act), 1.0f, 0.0f, 1, \
                       (float*)nullptr, (int)((M + 15) / 16));                                                      \
    break;
  switch ((L.rank + 15) / 16) {
    K1D_CASE(1) K1D_CASE(2) K1D_CASE(3) K1D_CASE(4) K1D_CASE(5) K1D_CASE(6) K1D_CASE(7) K1D_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef K1D_CASE
  return hipGetLastError();
}

hipError_t launch_k1(const KernelLayer& L, int64_t M, const uint16_t* X, int64_t ldx, uint8_t* qX,
                     void* sX, void* lora_act, bool mma, hipStream_t st, int parts, float* part_out, int full) {
  if (L.fmt == 0)
    return mma ? launch_k1_fmt<0, true>(L, M, X, ldx, qX, sX, lora_act, parts, part_out, full, st)
               : launch_k1_fmt<0, false>(L, M, X, ldx, qX, sX, lora_act, parts, part_out, full, st);
  if (L.fmt == 2)
    return mma ? launch_k1_fmt<2, true>(L, M, X, ldx, qX, sX, lora_act, parts, part_out, full, st)
               : launch_k1_fmt<2, false>(L, M, X, ldx, qX, sX, lora_act, parts, part_out, full, st);
  return mma ? launch_k1_fmt<1, true>(L, M, X, ldx, qX, sX, lora_act, parts, part_out, full, st)
             : launch_k1_fmt<1, false>(L, M, X, ldx, qX, sX, lora_act, parts, part_out, full, st);
}

K1Cut k1_cut(const KernelLayer& L, int64_t M) {
  // Long K: every block of 16 tokens walks many chunks, and the blocks past one per CU
  // double the time of the CUs that hold them; cut into 4 parts, every CU holds about the
  // same number of part blocks.  Short K at rank 0 (no sums to add across the parts) with
  // a last, partly filled round of one block per CU (the FLUX.1 layers' 4608 tokens: 288
  // blocks on 256 CUs): the blocks of the full rounds stay whole and only the last
  // round's blocks are cut, into as many parts (at most 8, at least one chunk each) as fit
  // one part block per CU beside the others.  At short K and rank > 0 the second step
  // (~5 us) costs as much as the balance gains, so kernel 1 runs in one pass.
  const int64_t nb = (M + 15) / 16;
  K1Cut c{(int)nb, 1};
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                               hipSuccess || cus < 1)
    return c;
  if (L.K >= 8192) {
    if (nb <= 2 * (int64_t)cus) c = K1Cut{0, 4};
    return c;
  }
  const int64_t rem = nb % cus;
  if (L.rank > 0 || nb < cus || rem == 0 || 2 * rem > cus) return c;
  int p = (int)(cus / rem) < 8 ? (int)(cus / rem) : 8;
  if (p > L.K / 64) p = (int)(L.K / 64);  // at least one chunk per range
  if (p < 2) return c;
  return K1Cut{(int)(nb - rem), p};
}

int k1_parts(const KernelLayer& L, int64_t M) { return k1_cut(L, M).parts; }

}  // namespace svdq
