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
//  * INT4: a sign-magnitude code q becomes the FP6 E2M3 field (sign, exponent 0,
//    mantissa |q|), whose value is q / 8 (a subnormal; exact), so an MFMA with block
//    scales 2^3 (E8M0 byte 130) on both sides yields the exact integer group sum I in
//    fp32, at the FP6 rate.  The per-group rescale: a second MFMA
//    (v_mfma_f32_32x32x8_f16) whose only nonzero k term is the pair of fp16 scales
//    forms c = s_X s_W for the 32 x 32 tile exactly (11 x 11 significant bits) in the
//    accumulator layout, and one v_fmac_f32 per output adds I * c.  The weight codes
//    come in a bit order from which masks alone give the FP6 operand words (prepared
//    once, offline).  In the forward the activation side comes from kernel 1 already in
//    operand form (FP6 words, fp16 scales, bf16 hi/lo low-rank activations), so the main
//    loop expands only the weights.
//
//  * NVFP4 (group 16, E4M3 scales under fp32 tensor scales): the scaled conversions take
//    only a scale's exponent and the block-scaled MFMA only E8M0 per 32, so each code
//    group is dequantized to fp16 in registers (exact) for v_mfma_f32_32x32x16_f16; the
//    two tensor scales multiply the 4-bit sum once after the loop.
//
// Tiling: 64-wide waves own TI x TJ MFMA tiles of 32 x 32 (SShape: INT4 4 x 1 of a
// 128 x 128 block, MXFP4 4 x 2 of 256 x 128, NVFP4 2 x 2 of 128 x 128; the packed-form
// kernel 2 x 2); two blocks share a CU, so one block's barrier and staging overlap
// another's math.  K advances in stages of 64-wide sub-steps, one barrier per stage.
// Two kernels implement this:
//  * k2_stream (MMA activation form, the forward's path): both operand panels and
//    their scales go global -> LDS with LDS-destination buffer loads into three
//    rotating buffers, loads for stage k+2 in flight while stage k is computed; the
//    weight codes stay 4-bit in LDS and each wave expands its own fragments.  Its DEBUG
//    instance runs the same loads, LDS layout, expansion and group-sum MFMA and stores
//    each group's MFMA result instead of rescaling it (the exact group sums); its CHAIN
//    instance (the MLP pair) runs the next layer's kernel 1 on the finished tile instead
//    of storing it (chain_epilogue).
//  * k2_gemm (packed activation form): 128 x 128 tiles of 4 waves; loads into registers
//    one stage ahead, converts the activation nibbles to FP6 operand words on the way
//    into double-buffered, row-padded LDS.
// Buffer resources' range checks return zeros past the end of either matrix, so no
// loop has bounds branches.  The tiles of a last, partly filled round of resident
// blocks are split along K; their partial tiles are summed by k2_fixup.
//
// 32x32x64 operand layout (measured): lane l supplies row/column l & 31; for FP4 it
// holds the 32 consecutive K values 32*(l>>5).. with the block scale of that half; for
// FP6 the fields of a lane half pair field f of A with field f of B, so A and B only
// need the same k order.  Output: lane l holds column l & 31, rows 8*(a>>2) + 4*(l>>5) +
// (a&3) for accumulator a = 0..15.
#include <type_traits>

#include "common.hpp"
#include "k1_parts.hpp"
#include "kernels.hpp"

namespace svdq {

namespace {

constexpr int BM = 128, BN = 128, NTHREADS = 256;
constexpr int WM = 64, WN = 64;  // wave tile; waves form a 2 x 2 grid
constexpr int TI = WM / 32, TJ = WN / 32;

template <int FMT, int SUB>
struct Smem {
  // operand bytes per row and 64-wide sub-step: INT4 holds each 32-code half as its six
  // FP6 operand words in two 16-byte slots (words 0-2 | pad, 3-5 | pad)
  static constexpr int kSub = FMT == 0 ? 64 : 32;
  static constexpr int kPitch = SUB * kSub + 16;
  // one stage's panels and scales
  struct Stage {
    uint16_t m[FMT == 0 ? SUB : 1][BM + BN];  // INT4 fp16 scale bits: X rows, then W columns
    uint32_t e[FMT == 0 ? 1 : SUB][BM + BN];  // MXFP4 E8M0 bytes (the sub-step's two groups in bytes 0, 1)
    uint8_t A[BM * kPitch];
    uint8_t B[BN * kPitch];
  } st[2];
};

// Store one 32 x 32 accumulator (rows r_off.., columns c_off.. of the tile at m0, n0)
// to Y (ydtype 0: fp32, 1: bf16, 2: bf16 of GELU(y)) through a resource over the
// tile's rows: rows past the end fall outside the range and are dropped; columns past N are masked (they may be the caller's row padding).
// The host guarantees (tile rows) * ldy * (element size) < 2^32 for every tile shape
// (ldy < 2^22 elements).
__device__ __forceinline__ void store_sub(const v16f& acc, void* Y, int64_t ldy, int ydtype, int64_t m0,
                                          int64_t n0, int64_t rowsA, int64_t nlim, int r_off, int c_off,
                                          int l32, int kh) {
  if (n0 + c_off + l32 >= nlim) return;
  const uint32_t ysz = ydtype == 0 ? 4u : 2u;
  const uint32_t ystep = (uint32_t)ldy * ysz;
  // base: element (m0, n0); range: to the end of row m0 + rowsA - 1
  const __amdgpu_buffer_rsrc_t rY = make_rsrc(static_cast<uint8_t*>(Y) + (m0 * ldy + n0) * ysz,
                                              (uint32_t)rowsA * ystep - (uint32_t)n0 * ysz);
  const uint32_t o = (uint32_t)(r_off + 4 * kh) * ystep + (uint32_t)(c_off + l32) * ysz;
  if (ydtype == 0) {
#pragma unroll
    for (int a = 0; a < 16; ++a)
      buf_store4(__float_as_uint(acc[a]), rY, o + (uint32_t)(8 * (a >> 2) + (a & 3)) * ystep);
  } else if (ydtype == 1) {
#pragma unroll
    for (int a = 0; a < 16; ++a)
      buf_store2((uint16_t)f32_to_bf16_rne(acc[a]), rY, o + (uint32_t)(8 * (a >> 2) + (a & 3)) * ystep);
  } else {  // bf16 of GELU(y), converted as in the chained epilogue
#pragma unroll
    for (int a = 0; a < 16; a += 2) {
      const uint32_t g2 = gelu_bf16x2(acc[a], acc[a + 1]);
      buf_store2((uint16_t)g2, rY, o + (uint32_t)(8 * (a >> 2) + (a & 3)) * ystep);
      buf_store2((uint16_t)(g2 >> 16), rY, o + (uint32_t)(8 * (a >> 2) + (a & 3) + 1) * ystep);
    }
  }
}

// Work split of one launch (see launch_k2): blocks [0, full) compute tiles 0 .. full-1
// over the whole K; the remaining tiles full .. are each cut into `split` parts along K,
// one block per part, which write fp32 partial tiles that k2_fixup adds up.
struct K2Sched {
  uint32_t tiles_n;  // tiles along N
  uint32_t full;     // tiles computed whole
  uint32_t split;    // parts per remaining tile (1: none remain)
  float* partials;   // [remaining * split][16 sub-tiles][16][64] fp32
};
// One partial tile: the 16 32 x 32 sub-tiles of the 128 x 128 tile, sub-tile (r, c) (row
// block r, column block c) at index 4 r + c, each 16 x 64 floats in the MFMA's lane
// layout (accumulator a of lane l at a * 64 + l).
constexpr int PART_FLOATS = 16 * 16 * 64;
static_assert(TI == 2 && TJ == 2, "the rescale schedules assume a 2 x 2 wave tile");

// One stage's global loads of one thread: 16-byte pieces of 4-bit codes.
template <int SUB>
struct Stage {
  uint4 a[2 * SUB], b[SUB];
  uint32_t s[SUB];
};

// The packed activation form: 4-bit codes [M][K/2] (INT4 nibbles are converted to FP6
// operand words on the way into LDS, the weights' prepared words expanded), scales
// [K/G][M] (INT4 fp16), lora_act fp32 [M][R16]; prepared weights (INT4 scales fp16).
template <int FMT, bool DEBUG, int SUB>
__global__ __launch_bounds__(NTHREADS, 2) __attribute__((amdgpu_waves_per_eu(2, 2))) void k2_gemm(
    const uint8_t* __restrict__ qX, const void* __restrict__ sXv, int64_t M,
    const uint8_t* __restrict__ qW, const void* __restrict__ sWv, int64_t N, int64_t K,
    const void* __restrict__ lora_act, const uint16_t* __restrict__ L2, int rank,
    void* __restrict__ Y, int64_t ldy, int ydtype,
    int64_t mbase, int64_t nbase, int64_t mlim, int64_t nlim, K2Sched sch, int32_t* __restrict__ dbg) {
  using S = Smem<FMT, SUB>;
  __shared__ S sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar
  const int l32 = lane & 31;
  const int kh = lane >> 5;
  const int wm = (wave >> 1) * WM;
  const int wn = (wave & 1) * WN;
  const uint32_t Kb = (uint32_t)(K >> 1);      // bytes per 4-bit code row
  const uint32_t Ka = Kb;                      // bytes per A row
  const int nstages = (int)(K >> 6) / SUB;     // the host picks SUB dividing K / 64
  // tile and stage range of this block; part < 0: the whole K
  uint32_t t = blockIdx.x;
  int part = -1, kbeg = 0, kend = nstages;
  if (t >= sch.full) {
    const uint32_t u = t - sch.full;
    t = sch.full + u / sch.split;
    part = (int)(u % sch.split);
    kbeg = (int)(((uint32_t)part * nstages) / sch.split);
    kend = (int)(((uint32_t)(part + 1) * nstages) / sch.split);
  }
  const int64_t m0 = mbase + (int64_t)(t / sch.tiles_n) * BM;
  const int64_t n0 = nbase + (int64_t)(t % sch.tiles_n) * BN;

  // ---- buffer resources (range-checked loads) -------------------------------------
  const int64_t rowsA = mlim - m0 < BM ? mlim - m0 : BM;
  const int64_t rowsB = nlim - n0 < BN ? nlim - n0 : BN;
  const __amdgpu_buffer_rsrc_t rA = make_rsrc(qX + m0 * Ka, (uint32_t)rowsA * Ka);
  // The prepared weights come in column pairs (two columns' 64-byte stage segments per
  // 128-byte line), addressed from the start of the array (the debug window may start at
  // an odd column); the range covers the pair of a last odd column
  const __amdgpu_buffer_rsrc_t rB = make_rsrc(qW, (uint32_t)((N + 1) & ~int64_t(1)) * Kb);
  const int ng = FMT == 0 ? (int)(K >> 6) : (int)(K >> 5);  // scale groups along K
  // staging roles: thread t moves the pieces of row t & 127, half t >> 7, of the A and
  // the B panel, and one scale per sub-step: waves 0-1 of the X row t, waves 2-3 of the
  // W column t - 128.  The choice is wave-uniform, so it is made once, here.
  const bool xs = wave < 2;
  // scale rows: the activation scales have stride M, the prepared weight scales are
  // padded to a multiple of 4; INT4: fp16, MXFP4: E8M0 bytes
  const uint32_t sstride = xs ? (uint32_t)M : (uint32_t)((N + 3) & ~int64_t(3));
  const uint32_t ssz = FMT == 0 ? 2u : 1u;
  const __amdgpu_buffer_rsrc_t rS = make_rsrc(xs ? sXv : sWv, DEBUG ? 0u : (uint32_t)ng * sstride * ssz);
  const uint32_t sidx = xs ? (uint32_t)(m0 + tid) : (uint32_t)(n0 + tid - BM);
  const int ldrow = tid & 127, ldhalf = tid >> 7;
  // this thread's part of a stage row: 4-bit code bytes [SUB*16*half, +SUB*16); in LDS,
  // INT4 takes 32 bytes per 32-code half (its FP6 operand words)
  // column pairs: byte b of column c at (c / 2) 2 Kb + (b / 64) 128 + (c % 2) 64 + b % 64
  // (a thread's pieces of a stage never cross a 64-byte segment)
  const uint32_t cB = (uint32_t)(n0 + ldrow);  // absolute column
  const uint32_t offB = (cB >> 1) * 2 * Kb + (cB & 1) * 64 + ldhalf * SUB * 16;
  const uint32_t offA = (uint32_t)ldrow * Ka + ldhalf * SUB * 16;
  const int ldsAB = ldrow * S::kPitch + ldhalf * SUB * (FMT == 0 ? 32 : 16);

  // Loads for stages past the end are harmless: they read zeros (range check) or codes
  // of another row into registers that are never stored.
  auto gload = [&](Stage<SUB>& st, int k) {
    const uint32_t kb = (uint32_t)k * SUB * 32;  // 4-bit code bytes before stage k
    const uint32_t kbB = (kb >> 6) * 128 + (kb & 63);
#pragma unroll
    for (int v = 0; v < SUB; ++v) {
      st.a[v] = buf_load16(rA, offA + kb + v * 16);
      st.b[v] = buf_load16(rB, offB + kbB + v * 16);
    }
#pragma unroll
    for (int u = 0; u < SUB; ++u) {
      const uint32_t g = (uint32_t)(k * SUB + u);  // 64-wide sub-step
      if (DEBUG) {
        st.s[u] = 0;
      } else if (FMT == 0) {
        st.s[u] = buf_load2(rS, (g * sstride + sidx) * 2);
      } else {
        const uint32_t o0 = 2 * g * sstride + sidx;
        st.s[u] = buf_load1(rS, o0) | (buf_load1(rS, o0 + sstride) << 8);
      }
    }
  };
  auto sstore = [&](const Stage<SUB>& st, int buf) {
    uint8_t* A = &sm.st[buf].A[ldsAB];
    uint8_t* B = &sm.st[buf].B[ldsAB];
#pragma unroll
    for (int v = 0; v < SUB; ++v) {
      if (FMT == 0) {
        const v6i fa = nib32_to_fp6(st.a[v]);
        const v8i fb = expand_w6(st.b[v]);
        uint4* da = reinterpret_cast<uint4*>(A + v * 32);
        uint4* db = reinterpret_cast<uint4*>(B + v * 32);
        da[0] = make_uint4(fa[0], fa[1], fa[2], 0u);
        da[1] = make_uint4(fa[3], fa[4], fa[5], 0u);
        db[0] = make_uint4(fb[0], fb[1], fb[2], 0u);
        db[1] = make_uint4(fb[3], fb[4], fb[5], 0u);
      } else {
        *reinterpret_cast<uint4*>(A + v * 16) = st.a[v];
        *reinterpret_cast<uint4*>(B + v * 16) = st.b[v];
      }
    }
#pragma unroll
    for (int u = 0; u < SUB; ++u) {
      if (FMT == 0) {
        sm.st[buf].m[u][tid] = (uint16_t)st.s[u];
      } else {
        sm.st[buf].e[u][tid] = st.s[u];
      }
    }
  };

  v16f acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = v16f{};

  // one 64-wide sub-step u of the stage in LDS buffer buf (global index g for the debug
  // output)
  auto compute = [&](int buf, int u, int g) {
    v8i bf[TJ], af[TI];
    uint32_t sb[TJ], sa[TI];
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int col = wn + j * 32 + l32;
      if (FMT == 0) {
        const uint4* p = reinterpret_cast<const uint4*>(&sm.st[buf].B[col * S::kPitch + u * 64 + kh * 32]);
        const uint4 x0 = p[0], x1 = p[1];
        bf[j] = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x1.x, (int)x1.y, (int)x1.z, 0, 0};
        const uint32_t w = sm.st[buf].m[u][BM + col];
        sb[j] = kh ? 0u : w;  // the column scale enters the scale product once (k = 0)
      } else {
        const uint4 x0 = *reinterpret_cast<const uint4*>(&sm.st[buf].B[col * S::kPitch + u * 32 + kh * 16]);
        bf[j] = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, 0, 0, 0, 0};
        sb[j] = (sm.st[buf].e[u][BM + col] >> (8 * kh)) & 0xFF;
      }
    }
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const int row = wm + i * 32 + l32;
      if (FMT == 0) {
        const uint4* p = reinterpret_cast<const uint4*>(&sm.st[buf].A[row * S::kPitch + u * 64 + kh * 32]);
        const uint4 x0 = p[0], x1 = p[1];
        af[i] = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x1.x, (int)x1.y, (int)x1.z, 0, 0};
        sa[i] = sm.st[buf].m[u][row];
      } else {
        const uint4 x0 = *reinterpret_cast<const uint4*>(&sm.st[buf].A[row * S::kPitch + u * 32 + kh * 16]);
        af[i] = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, 0, 0, 0, 0};
        sa[i] = (sm.st[buf].e[u][row] >> (8 * kh)) & 0xFF;
      }
    }
    if (FMT == 0) {
      // FP6 codes q / 8 with block scales 2^3 on both sides: the exact integer group sum
      auto gs = [&](int i, int j) {
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bf[j], v16f{}, 2, 2, 0, 130, 0, 130);
      };
      // c = sX sW for the tile, exact (see k2_stream)
      auto sc = [&](int i, int j) {
        const v4h a = __builtin_bit_cast(v4h, make_uint2(sa[i], 0u));
        const v4h b = __builtin_bit_cast(v4h, make_uint2(sb[j], 0u));
        return __builtin_amdgcn_mfma_f32_32x32x8f16(a, b, v16f{}, 0, 0, 0);
      };
      if (DEBUG) {
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
          for (int j = 0; j < TJ; ++j) {
            const v16f p = gs(i, j);
#pragma unroll
            for (int a = 0; a < 16; ++a) {
              const int64_t r = m0 + wm + i * 32 + 8 * (a >> 2) + 4 * kh + (a & 3);
              const int64_t c = n0 + wn + j * 32 + l32;
              if (r < mlim && c < nlim)
                dbg[((int64_t)g * (mlim - mbase) + (r - mbase)) * (nlim - nbase) + (c - nbase)] = (int32_t)p[a];
            }
          }
      } else {
        auto epi = [&](int i, int j, const v16f& p, const v16f& c) {
#pragma unroll
          for (int a = 0; a < 16; ++a) acc[i][j][a] = fmaf(p[a], c[a], acc[i][j][a]);
        };
        v16f c0 = sc(0, 0), p0 = gs(0, 0);
        v16f c1 = sc(0, 1), p1 = gs(0, 1);
        epi(0, 0, p0, c0);
        c0 = sc(1, 0);
        p0 = gs(1, 0);
        epi(0, 1, p1, c1);
        c1 = sc(1, 1);
        p1 = gs(1, 1);
        epi(1, 0, p0, c0);
        epi(1, 1, p1, c1);
      }
    } else {
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bf[j], acc[i][j], 4, 4, 0, (int)sa[i], 0,
                                                                     (int)sb[j]);
    }
  };

  // ---- main loop: the next stage's loads are issued first, LDS double buffer, one
  // barrier per stage ------------------------------------------------------------------
  Stage<SUB> r;
  gload(r, kbeg);
  sstore(r, 0);
  __syncthreads();
  for (int k = kbeg; k < kend; ++k) {
    const int buf = (k - kbeg) & 1;
    gload(r, k + 1);
#pragma unroll
    for (int u = 0; u < SUB; ++u) compute(buf, u, k * SUB + u);
    sstore(r, buf ^ 1);
    __syncthreads();
  }
  if (DEBUG) return;

  // ---- low-rank up projection: acc += lora_act[rows, :] L2[:, cols] -------------------
  // v_mfma_f32_32x32x16_bf16 with a bf16 hi/lo split of lora_act (L2 is bf16 already).
  // lora_act is [M][R16] fp32 (lane (row l & 31, kh) reads the 8 consecutive ranks
  // 16 t + 8 kh..), L2f is in fragment order (one 16-byte piece per lane, 1 KB per
  // column block and k step); rows past M / columns past N read as zeros through the
  // range check.
  if (rank > 0 && part <= 0) {  // once per tile: whole, or the first part
    const int R16 = (rank + 15) & ~15;
    const __amdgpu_buffer_rsrc_t rL = make_rsrc(static_cast<const uint8_t*>(lora_act) + m0 * R16 * 4, (uint32_t)(rowsA * R16 * 4));
    const __amdgpu_buffer_rsrc_t rU = make_rsrc(L2 + n0 * R16, (uint32_t)(((rowsB + 31) & ~31) * R16 * 2));
    for (int k0 = 0; k0 < R16; k0 += 16) {
      v8bf bl[TJ];
#pragma unroll
      for (int j = 0; j < TJ; ++j)
        bl[j] = __builtin_bit_cast(v8bf, buf_load16(rU, (uint32_t)(((((wn >> 5) + j) * (R16 >> 4) + (k0 >> 4)) * 64 + lane) * 16)));
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        const uint32_t o = (uint32_t)((wm + i * 32 + l32) * R16 + k0 + 8 * kh) * 4;
        const uint4 v0 = buf_load16(rL, o), v1 = buf_load16(rL, o + 16);
        const float v[8] = {__uint_as_float(v0.x), __uint_as_float(v0.y), __uint_as_float(v0.z), __uint_as_float(v0.w),
                            __uint_as_float(v1.x), __uint_as_float(v1.y), __uint_as_float(v1.z), __uint_as_float(v1.w)};
        uint16_t hi[8], lo[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const uint32_t hb = f32_to_bf16_rne(v[u]);
          hi[u] = (uint16_t)hb;
          lo[u] = (uint16_t)f32_to_bf16_rne(v[u] - __uint_as_float(hb << 16));
        }
        const v8bf ah = __builtin_bit_cast(v8bf, hi);
        const v8bf al = __builtin_bit_cast(v8bf, lo);
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bl[j], acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bl[j], acc[i][j], 0, 0, 0);
        }
      }
    }
  }

  // ---- store (or the partial tile) ------------------------------------------------------
  if (part < 0) {
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j) store_sub(acc[i][j], Y, ldy, ydtype, m0, n0, rowsA, nlim, wm + i * 32, wn + j * 32, l32, kh);
  } else {
    float* P = sch.partials + (size_t)(blockIdx.x - sch.full) * PART_FLOATS;
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int st = ((wm >> 5) + i) * 4 + (wn >> 5) + j;
#pragma unroll
        for (int a = 0; a < 16; ++a) P[(st * 16 + a) * 64 + lane] = acc[i][j][a];
      }
  }
}

// ---------------------------------------------------------------------------------------
// Kernel 2, streamed (MMA activation form): codes and scales go from global memory
// straight into LDS with buffer loads that write LDS (each lane's 16 or 4 bytes land at
// the instruction's LDS base + lane * size): no register staging and no LDS store
// instructions.  Three LDS buffers rotate; a stage is two 64-wide sub-steps (K is a
// multiple of 128), and the loads of stage k+2 are in flight while stage k is computed,
// with one barrier per stage.
// 16-byte slots of each operand row are XOR-swizzled with the row (rows are not padded:
// a load instruction fills 1 KB contiguously).  The weight codes stay 4-bit in LDS and
// are expanded to FP6 operand words after the read, per wave (masks only).
// INT4 rescale: both MFMA block scales are 2^3, so the MFMA returns the exact integer
// group sum I; a second MFMA forms c = s_X s_W exactly and the epilogue adds I * c with
// one v_fmac_f32 per output and group.

// Block shape: a WGM x WGN grid of waves, each owning TI x TJ MFMA tiles of 32 x 32.
template <int WGM_, int WGN_, int TI_, int TJ_>
struct Shape {
  static constexpr int WGM = WGM_, WGN = WGN_, TI = TI_, TJ = TJ_;
  static constexpr int NW = WGM * WGN, NT = 64 * NW;
  static constexpr int BM = 32 * TI * WGM, BN = 32 * TJ * WGN;
  static constexpr int CB = BN / 32;                 // 32-wide column blocks per tile
  static constexpr int PART = (BM / 32) * CB * 16 * 64;  // floats per partial tile
};
// INT4: 128 x 128, 4 waves side by side, each 128 x 32 (four row tiles against one
// column tile), two blocks per CU (a 128 x 256 tile with one block per CU measured 6%
// slower: the waves of one block meet at every barrier).  The per-group rescale makes
// VALU work the bound; a wave expands one weight fragment per group for four tiles
// (half the expansion work of 64 x 64 waves, for a third more LDS operand reads).
// MXFP4: 256 x 128, 4 waves of 128 x 64, two blocks per CU (no per-group VALU, so larger
// wave tiles; measured against 256 x 256 tiles of 8 waves, which halve the panel bytes
// per output but leave the QKV layer 2.53 rounds of tiles in 3 rounds of one block per
// CU: 96 against 102 us).
// NVFP4: 128 x 128, 4 waves of 64 x 64; its matrix-core work is fp16 (four 16-deep
// MFMAs per 64 K, on operands dequantized in registers), which bounds it.
template <int FMT> struct SShape;
template <> struct SShape<0> : Shape<1, 4, 4, 1> {};
template <> struct SShape<2> : Shape<2, 2, 2, 2> {};
template <> struct SShape<1> : Shape<2, 2, 4, 2> {};

// LDS layout of one stage of the streamed kernel
template <int FMT>
struct DLay {
  using SH = SShape<FMT>;
  static constexpr int BM = SH::BM, BN = SH::BN, NW = SH::NW;
  static constexpr int RA = 2 * (FMT == 0 ? 64 : 32);  // A bytes per row
  static constexpr int RB = 2 * 32;                     // B (4-bit) bytes per row
  static constexpr int B_OFF = BM * RA;
  static constexpr int S_OFF = B_OFF + BN * RB;
  // scales of one sub-step: INT4 X [BM] fp16 | W [BN] fp16; MXFP4 X e [2][BM] | W e [2][BN]
  // (the sub-step's two 32-groups); NVFP4 X [BM][4] | W [BN][4] E4M3 (four 16-groups);
  // moved in 256-byte parts, one 4-byte load per lane
  static constexpr int SPR = FMT == 2 ? 4 : 2;  // scale bytes per row and sub-step
  static constexpr int XB = SPR * BM, WB = SPR * BN;
  static constexpr int S_SUB = XB + WB;
  static constexpr int XP = XB / 256, WP = WB / 256, SPARTS = 2 * (XP + WP);  // per stage
  static constexpr int NS = (SPARTS + NW - 1) / NW;  // scale loads per wave
  // slots past SPARTS load a part again into a spare 256 bytes, so every wave issues NS
  static constexpr int SPARE = S_OFF + 2 * S_SUB;
  static constexpr int BUF = SPARE + (NS * NW > SPARTS ? 256 : 0);
  // load instructions per wave and stage
  static constexpr int NA = BM * RA / 1024 / NW;
  static constexpr int NBW = BN * RB / 1024 / NW;
  static constexpr int NDW = NA + NBW + NS;
  static_assert(BM * RA % (1024 * NW) == 0 && BN * RB % (1024 * NW) == 0, "whole 1 KB load chunks per wave");
  static_assert(XB % 256 == 0 && WB % 256 == 0, "whole 256-byte scale parts");
};

// XOR swizzle of the 16-byte slot within a row of `slots` slots.  An operand read
// (ds_read_b128, one row per lane) is served 16 lanes, i.e. 16 consecutive rows, per
// pass over the 64 banks (256 bytes): the rows of one pass that share their position
// within 256 bytes must get different slots.  The functions also keep any 8
// consecutive rows apart within 128 bytes.  (Measured: no bank conflicts; the plain
// row & 7 / (row >> 1) & 3 patterns conflicted two ways.)
__device__ __forceinline__ int swz(int row, int slots) {
  return slots == 8 ? ((row ^ (row >> 3)) & 7) : (((row >> 1) ^ (row >> 2)) & 3);
}

// 16 bytes per lane global -> LDS; soff (wave-uniform) is added to the address: the
// range check on voff alone still drops every row past the end of the panel
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 4, off, 0, 0, 0);
}

// s_waitcnt vmcnt(N) and lgkmcnt(L) (expcnt untouched; L = 15: untouched)
template <int N, int L = 15>
__device__ __forceinline__ void wait_cnt() {
  static_assert(N >= 0 && N < 64 && L >= 0 && L < 16, "counter range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (L << 8));
}

// The DEBUG instance's output: the exact INT4 group sums I[g][r][c] of the window rows
// [m0, m0 + mt) x columns [n0, n0 + nt), int32 [K/64][mt][nt].
struct K2Debug {
  int32_t* out;
  int64_t m0, n0, mt, nt;
};

// The chained MLP pair: the CHAIN instance (INT4 fc1, whole tiles) turns its finished
// 128 x 128 tile H into fc2's activation side instead of storing it: G = bf16(GELU(H))
// through LDS, then kernel 1's steps on G (smoothing by fc2's 1 / s, INT4 group-64 codes
// and fp16 scales in the MMA form, down projection by fc2's L1).  The tile holds 128 of
// fc2's input channels, two whole groups of every row, so the per-token group scales are
// complete; the down projection over these 128 channels is a partial sum, stored per
// column tile and summed over the tiles in a fixed order by k2_lora_reduce.
struct K2Chain {
  uint8_t* qX2;           // fc2 codes, MMA form [M][K2] (K2 = fc1's N)
  uint16_t* sX2;          // fc2 fp16 scales [K2 / 64][Mp]
  float* part;            // down-projection partials [K2 / 128][M][16 nt2]
  const float* inv_s2;    // fc2 1 / s [K2]
  const uint16_t* L1f2;   // fc2 L1 in kernel 1's fragment order
  int nt2;                // fc2 rank tiles of 16
  uint16_t* hidden;       // optional copy of G, bf16 [M][ldh] (NULL: not written)
  int64_t ldh;
};

// Rows of a 64-channel half of the G tile in LDS: 128 bytes + 16, so the 16 rows read by
// one 16-lane pass of a ds_read_b128 start 4 banks apart (36 r mod 64 for rows r = 0..15:
// distinct multiples of 4).
constexpr int GPITCH = 144;

// The CHAIN instance's epilogue (see K2Chain).  acc: the INT4 wave tile (four 32 x 32
// tiles, rows 0..127 of the block, columns wn..wn+31), the finished H including fc1's
// low-rank term.  Steps:
//  1. G = bf16(GELU(H)), rows past M as 0, into LDS (channels 0-63 of the tile in lds0,
//     64-127 in lds1, GPITCH bytes per row), and into `hidden` when it is given;
//  2. wave w takes the tile's tokens 32 w .. 32 w + 31 as two blocks of 16, in kernel 1's
//     lane layout (lane l: token l & 15, channels 16 (l >> 4) .. +15 of a group), reads
//     G, smooths it by fc2's 1 / s, and runs kernel 1's INT4 quantizer and MMA-form word
//     builder and its bf16 hi / lo down projection;
//  3. the down projection over the tile's 128 channels goes to part[tile column][token]
//     (one 16-column rank tile at a time, so any fc2 rank runs in one instance).
__device__ __forceinline__ void chain_epilogue(const v16f (&acc)[4][1], const K2Chain& ch, int64_t M, int64_t K2,
                                               int64_t m0, int64_t n0, int64_t rowsA, uint8_t* lds0, uint8_t* lds1,
                                               int wave, int lane, int wn, int l32, int kh, uint32_t Mp) {
  // every wave has finished its reads of the last stage, and its own loads have landed
  __syncthreads();
  // Rows past M are not masked: their accumulators reach only those rows' own codes,
  // scales and down projections (per-token groups; MFMA rows are independent), none of
  // which is stored.  Two rows 8 q + j, 8 q + j + 1 share one bf16 conversion.
  uint8_t* gw = (wave < 2 ? lds0 : lds1) + ((wn & 63) + l32) * 2 + 4 * kh * GPITCH;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int a = 0; a < 16; a += 2) {
      const int r = i * 32 + 8 * (a >> 2) + (a & 3);
      const uint32_t g2 = gelu_bf16x2(acc[i][0][a], acc[i][0][a + 1]);
      *reinterpret_cast<uint16_t*>(gw + r * GPITCH) = (uint16_t)g2;
      *reinterpret_cast<uint16_t*>(gw + (r + 1) * GPITCH) = (uint16_t)(g2 >> 16);
    }
  __syncthreads();
  if (ch.hidden != nullptr) {  // the optional copy of G, 16 bytes per thread and step
    for (int e = wave * 64 + lane; e < 128 * 16; e += 256) {
      const int r = e >> 4, pc = e & 15;
      if (r < rowsA)
        *reinterpret_cast<uint4*>(ch.hidden + (m0 + r) * ch.ldh + n0 + 8 * pc) =
            *reinterpret_cast<const uint4*>((pc < 8 ? lds0 : lds1) + r * GPITCH + (pc & 7) * 16);
    }
  }

  const int r16 = lane & 15, sub = lane >> 4;
  const int64_t c0 = n0 >> 6;  // fc2's group (chunk) index of the tile's first half
  const __amdgpu_buffer_rsrc_t rI = make_rsrc(ch.inv_s2 + n0, 128u * 4u);
  float is[2][16];
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 v = buf_load16(rI, (uint32_t)((g * 64 + sub * 16 + 4 * q) * 4));
      is[g][4 * q] = __uint_as_float(v.x);
      is[g][4 * q + 1] = __uint_as_float(v.y);
      is[g][4 * q + 2] = __uint_as_float(v.z);
      is[g][4 * q + 3] = __uint_as_float(v.w);
    }
  const int nt2 = ch.nt2;
  const int64_t R16 = 16 * (int64_t)nt2;
  const __amdgpu_buffer_rsrc_t rL = make_rsrc(ch.L1f2, (uint32_t)(R16 * K2 * 2));
  float* part = ch.part + ((n0 >> 7) * M + m0) * R16;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int tb = (2 * wave + b) * 16;  // the token block's first row in the tile
    const int tr = tb + r16;
    const int64_t row = m0 + tr;
    float xh[2][16];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const uint8_t* src = (g ? lds1 : lds0) + tr * GPITCH + sub * 32;
      const uint4 p0 = *reinterpret_cast<const uint4*>(src), p1 = *reinterpret_cast<const uint4*>(src + 16);
      const uint32_t w[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        xh[g][2 * j] = bf16_lo_to_f32(w[j]) * is[g][2 * j];
        xh[g][2 * j + 1] = bf16_hi_to_f32(w[j]) * is[g][2 * j + 1];
      }
    }
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      float t[16];
      const _Float16 sh = int4_quantize16(xh[g], t);
      const uint4 mw = int4_mma_words(t, sub);  // every lane takes part in the swaps
      if (tr < rowsA) {
        *reinterpret_cast<uint4*>(ch.qX2 + row * K2 + n0 + g * 64 + sub * 16) = mw;
        if (sub == 0) ch.sX2[(c0 + g) * (int64_t)Mp + row] = __builtin_bit_cast(uint16_t, sh);
      }
    }
    // rank tiles two at a time (one hi / lo split of the activations per pair), a last
    // odd one alone
    auto tiles = [&](auto NTc, int t0) {
      constexpr int NT = decltype(NTc)::value;
      v4f la[NT];
#pragma unroll
      for (int u = 0; u < NT; ++u) la[u] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        uint4 LA[NT], LB[NT];
#pragma unroll
        for (int u = 0; u < NT; ++u) {
          const uint32_t o = (uint32_t)((((c0 + g) * nt2 + t0 + u) * 64 + lane) * 32);
          LA[u] = buf_load16(rL, o);
          LB[u] = buf_load16(rL, o + 16);
        }
        lora_down16<NT>(la, xh[g], LA, LB);
      }
      // each 16 x 16 result: lane l holds rank column 16 t + (l & 15), rows 4 (l >> 4) + i
#pragma unroll
      for (int u = 0; u < NT; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rr = tb + 4 * sub + i;
          if (rr < rowsA) part[rr * R16 + 16 * (t0 + u) + r16] = la[u][i];
        }
    };
    int t = 0;
    for (; t + 2 <= nt2; t += 2) tiles(std::integral_constant<int, 2>{}, t);
    if (t < nt2) tiles(std::integral_constant<int, 1>{}, t);
  }
}

template <int FMT, bool DEBUG = false, bool CHAIN = false>
__global__ __launch_bounds__(SShape<FMT>::NT, 8 / SShape<FMT>::NW) __attribute__((amdgpu_waves_per_eu(2, 2))) void k2_stream(
    const uint8_t* __restrict__ qX, const uint8_t* __restrict__ sX, int64_t M,
    const uint8_t* __restrict__ qW, const uint8_t* __restrict__ sW, int64_t N, int64_t K,
    const uint16_t* __restrict__ lora_act, const uint16_t* __restrict__ L2, int rank,
    void* __restrict__ Y, int64_t ldy, int ydtype, K2Sched sch, K2Debug dbg, float sxw, K2Chain ch) {
  static_assert(!DEBUG || FMT == 0, "group sums are defined for INT4");
  static_assert(!CHAIN || (FMT == 0 && !DEBUG), "the chained epilogue follows the INT4 layer");
  // NVFP4: sxw = fp32(S_X S_W), the product of the two tensor scales
  using D = DLay<FMT>;
  using SH = SShape<FMT>;
  constexpr int TI = SH::TI, TJ = SH::TJ, BM = SH::BM, BN = SH::BN, NW = SH::NW;
  // separate arrays, always addressed statically (the main loop is unrolled by 3), so
  // the compiler can tell a buffer's pending loads from reads of another
  __shared__ __attribute__((aligned(1024))) uint8_t lds0[D::BUF];
  __shared__ __attribute__((aligned(1024))) uint8_t lds1[D::BUF];
  __shared__ __attribute__((aligned(1024))) uint8_t lds2[D::BUF];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int kh = lane >> 5;
  const int wm = (wave / SH::WGN) * (32 * TI);
  const int wn = (wave % SH::WGN) * (32 * TJ);
  const uint32_t Kb = (uint32_t)(K >> 1);                  // 4-bit code bytes per row
  const uint32_t Ka = FMT == 0 ? (uint32_t)K : Kb;         // A bytes per row
  const int nstages = (int)(K >> 7);
  uint32_t t = blockIdx.x;
  int part = -1, kbeg = 0, kend = nstages;
  if (t >= sch.full) {
    const uint32_t u = t - sch.full;
    t = sch.full + u / sch.split;
    part = (int)(u % sch.split);
    kbeg = (int)(((uint32_t)part * nstages) / sch.split);
    kend = (int)(((uint32_t)(part + 1) * nstages) / sch.split);
  }
  const int64_t m0 = (int64_t)(t / sch.tiles_n) * BM;
  const int64_t n0 = (int64_t)(t % sch.tiles_n) * BN;
  const int64_t rowsA = M - m0 < BM ? M - m0 : BM;
  const int64_t rowsB = N - n0 < BN ? N - n0 : BN;
  // Row pairs: the weights (both formats) and the MXFP4 activations keep the 64-byte stage
  // segments of rows 2j, 2j+1 in one 128-byte line; the ranges cover a last odd row's pair
  const __amdgpu_buffer_rsrc_t rA = make_rsrc(qX + m0 * Ka, (uint32_t)(FMT != 0 ? (rowsA + 1) & ~int64_t(1) : rowsA) * Ka);
  const __amdgpu_buffer_rsrc_t rB = make_rsrc(qW + n0 * Kb, (uint32_t)((rowsB + 1) & ~int64_t(1)) * Kb);
  const uint32_t ng = FMT == 0 ? (uint32_t)(K >> 6) : (FMT == 1 ? (uint32_t)(K >> 5) : (uint32_t)(K >> 4));
  const uint32_t Mp = (uint32_t)((M + 3) & ~int64_t(3)), Np = (uint32_t)((N + 3) & ~int64_t(3));
  // DEBUG: no scales (empty ranges: the scale loads return zeros and touch no memory)
  const __amdgpu_buffer_rsrc_t rSX = make_rsrc(sX, DEBUG ? 0u : ng * Mp * (FMT == 0 ? 2 : 1));
  const __amdgpu_buffer_rsrc_t rSW = make_rsrc(sW, DEBUG ? 0u : ng * Np * (FMT == 0 ? 2 : 1));

  // ---- loads of stage k into an LDS buffer (every wave issues D::NDW instructions) ------
  // Per-lane source offsets within a stage are fixed (chunk n of 1 KB covers rows
  // n * 1024 / R ..); the stage's offset along K goes in the scalar offset.
  uint32_t voA[D::NA], voB[D::NBW];
#pragma unroll
  for (int q = 0; q < D::NA; ++q) {
    const int pos = (wave + NW * q) * 1024 + lane * 16;
    const int row = pos / D::RA, ps = (pos % D::RA) / 16;
    const uint32_t sl = (uint32_t)((ps ^ swz(row, D::RA / 16)) * 16);
    voA[q] = FMT != 0 ? (uint32_t)(row >> 1) * 2 * Ka + (uint32_t)(row & 1) * D::RA + sl : (uint32_t)row * Ka + sl;
  }
#pragma unroll
  for (int q = 0; q < D::NBW; ++q) {
    const int pos = (wave + NW * q) * 1024 + lane * 16;
    const int row = pos / D::RB, ps = (pos % D::RB) / 16;
    const uint32_t sl = (uint32_t)((ps ^ swz(row, D::RB / 16)) * 16);
    voB[q] = (uint32_t)(row >> 1) * 2 * Kb + (uint32_t)(row & 1) * D::RB + sl;
  }
  auto issue = [&](int k, uint8_t* base) {
#pragma unroll
    for (int q = 0; q < D::NA; ++q) dma16(rA, base + (wave + NW * q) * 1024, voA[q], (uint32_t)k * (FMT != 0 ? 2 : 1) * D::RA);
#pragma unroll
    for (int q = 0; q < D::NBW; ++q)
      dma16(rB, base + D::B_OFF + (wave + NW * q) * 1024, voB[q], (uint32_t)k * 2 * D::RB);
    // scale parts: slot z = wave + NW r covers sub-step z / (XP + WP), part y of it
    // (activation parts first); slots past the last part reload part 0 of sub-step 0
    // into the spare bytes.  Everything is wave-uniform arithmetic (no branches, so the
    // compiler keeps tracking which buffer has loads pending).
#pragma unroll
    for (int r = 0; r < D::NS; ++r) {
      const int z0 = wave + NW * r;
      const bool spare = z0 >= D::SPARTS;
      const int z = spare ? 0 : z0;
      const int u = z / (D::XP + D::WP), y = z % (D::XP + D::WP);
      const bool wside = y >= D::XP;
      const int yp = wside ? y - D::XP : y;
      uint8_t* dst = spare ? base + D::SPARE : base + D::S_OFF + u * D::S_SUB + (wside ? D::XB : 0) + yp * 256;
      const uint32_t pitch = wside ? Np : Mp, org = wside ? (uint32_t)n0 : (uint32_t)m0;
      const uint32_t g = (uint32_t)(k * 2 + u);
      uint32_t off;
      if (FMT == 0) {  // fp16 values of rows yp * 128 + 2 lane, + 1
        off = (g * pitch + org) * 2 + (uint32_t)(yp * 256 + lane * 4);
      } else if (FMT == 2) {  // [K/64][pitch][4]: the four E4M3 scales of row yp * 64 + lane
        off = (g * pitch + org) * 4 + (uint32_t)(yp * 256 + lane * 4);
      } else {  // bytes [gi][row] of the [2][B] region: byte yp * 256 + 4 lane ..
        const int bpg = wside ? BN : BM;
        const int b0 = yp * 256 + lane * 4;
        off = (2 * g + (uint32_t)(b0 / bpg)) * pitch + org + (uint32_t)(b0 % bpg);
      }
      dma4(wside ? rSW : rSX, dst, off);
    }
  };

  v16f acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = v16f{};

  // ---- the fragments of one sub-step u of a stage, read from LDS --------------------------
  struct Frag {
    uint4 a[TI];                    // A: INT4 FP6 operand words 0-3 (4-5 in a4), MXFP4 32 nibbles
    uint2 a4[FMT == 0 ? TI : 1];    // A: INT4 FP6 operand words 4-5
    uint4 b[TJ];                    // B: 32 4-bit codes
    uint32_t sa[TI], sb[TJ];        // MXFP4: E8M0 block scales; INT4: fp16 scale bits of the
                                    // lane's row / column (the column's 0 in lanes 32-63)
  };
  auto load = [&](const uint8_t* base, int u, Frag& f) {
    const uint8_t* sb = base + D::S_OFF + u * D::S_SUB;
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int col = wn + j * 32 + l32;
      const int ls = u * 2 + kh;  // 4-bit bytes u*32 + kh*16
      f.b[j] = *reinterpret_cast<const uint4*>(base + D::B_OFF + col * D::RB + ((ls ^ swz(col, D::RB / 16)) * 16));
      if constexpr (FMT == 0) {
        const uint32_t w = reinterpret_cast<const uint16_t*>(sb + D::XB)[col];
        f.sb[j] = kh ? 0u : w;
      } else if constexpr (FMT == 2) {
        f.sb[j] = reinterpret_cast<const uint32_t*>(sb + D::XB)[col];  // the column's four E4M3 scales
      } else {
        f.sb[j] = sb[D::XB + kh * BN + col];
      }
    }
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const int row = wm + i * 32 + l32;
      if constexpr (FMT == 0) {
        // operand half kh of sub-step u: bytes u*64 + kh*32 in two slots, [w0 w1 w2 w3 |
        // w4 w5 0 0]: a 16-byte and an 8-byte read into one aligned run of registers
        const int ls0 = u * 4 + kh * 2;
        const int sw = swz(row, D::RA / 16);
        f.a[i] = *reinterpret_cast<const uint4*>(base + row * D::RA + ((ls0 ^ sw) * 16));
        f.a4[i] = *reinterpret_cast<const uint2*>(base + row * D::RA + (((ls0 + 1) ^ sw) * 16));
        f.sa[i] = reinterpret_cast<const uint16_t*>(sb)[row];
      } else {
        const int ls = u * 2 + kh;
        f.a[i] = *reinterpret_cast<const uint4*>(base + row * D::RA + ((ls ^ swz(row, D::RA / 16)) * 16));
        if constexpr (FMT == 2) f.sa[i] = reinterpret_cast<const uint32_t*>(sb)[row];
        else f.sa[i] = sb[kh * BM + row];
      }
    }
  };

  // ---- INT4: weight expansion, group-sum MFMA, scale products, rescale -------------------
  auto expand = [&](const Frag& f, v8i (&bf)[TJ]) {
#pragma unroll
    for (int j = 0; j < TJ; ++j) bf[j] = expand_w6(f.b[j]);
  };
  // FP6 code q is q / 8 and both block scales are 2^3 (E8M0 byte 130), so the MFMA
  // returns the exact integer group sum I
  auto gs = [&](const Frag& f, const v8i (&bf)[TJ], int i, int j) {
    const uint4 x0 = f.a[i];
    const uint2 x1 = f.a4[FMT == 0 ? i : 0];
    const v8i af = {(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af, bf[j], v16f{}, 2, 2, 0, 130, 0, 130);
  };
  // c = sX sW for the 32 x 32 tile: an fp16 MFMA whose only nonzero k term is the pair of
  // scales (k = 0 in lanes 0-31; the column scale is 0 in lanes 32-63), so every
  // product is exact in fp32 (11 + 11 significant bits) and c has the accumulator layout
  auto sc = [&](const Frag& f, int i, int j) {
    const v4h a = __builtin_bit_cast(v4h, make_uint2(f.sa[i], 0u));
    const v4h b = __builtin_bit_cast(v4h, make_uint2(f.sb[j], 0u));
    return __builtin_amdgcn_mfma_f32_32x32x8f16(a, b, v16f{}, 0, 0, 0);
  };
  // acc += I * c: one rounding per group, the same value as (I * sW) * sX with the exact
  // product I * sW
  auto epi = [&](int i, int j, const v16f& p, const v16f& c) {
#pragma unroll
    for (int a = 0; a < 16; ++a) acc[i][j][a] = fmaf(p[a], c[a], acc[i][j][a]);
  };
  // ---- MXFP4: the MFMA accumulates the block-scaled products directly ---------------------
  auto mma4 = [&](const Frag& f) {
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const v8i af = {(int)f.a[i].x, (int)f.a[i].y, (int)f.a[i].z, (int)f.a[i].w, 0, 0, 0, 0};
        const v8i bf = {(int)f.b[j].x, (int)f.b[j].y, (int)f.b[j].z, (int)f.b[j].w, 0, 0, 0, 0};
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af, bf, acc[i][j], 4, 4, 0, (int)f.sa[i], 0,
                                                                   (int)f.sb[j]);
      }
  };

  // ---- NVFP4: dequantize to fp16 in registers, fp16 MFMA --------------------------------
  // K step s (16 deep) of the sub-step is group s: the lane's 16 bytes hold, per s, the
  // four bytes of its eight codes k = 16 s + 8 kh .. +7 (the MMA-form lane order), and
  // nv_f16x8 turns them into e2m1 * s_g in fp16, exact, so the MFMA accumulates exact
  // products.
  auto mma_nv_step = [&](const Frag& f, auto S) {
    constexpr int s = decltype(S)::value;
    v8h ab[TI], bb[TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const float sc = __builtin_amdgcn_cvt_f32_fp8((int)f.sa[i], s);
      const uint32_t w = s == 0 ? f.a[i].x : s == 1 ? f.a[i].y : s == 2 ? f.a[i].z : f.a[i].w;
      ab[i] = nv_f16x8(w, sc);
    }
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const float sc = __builtin_amdgcn_cvt_f32_fp8((int)f.sb[j], s);
      const uint32_t w = s == 0 ? f.b[j].x : s == 1 ? f.b[j].y : s == 2 ? f.b[j].z : f.b[j].w;
      bb[j] = nv_f16x8(w, sc);
    }
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ab[i], bb[j], acc[i][j], 0, 0, 0);
  };
  auto mma_nv = [&](const Frag& f) {
    mma_nv_step(f, std::integral_constant<int, 0>{});
    mma_nv_step(f, std::integral_constant<int, 1>{});
    mma_nv_step(f, std::integral_constant<int, 2>{});
    mma_nv_step(f, std::integral_constant<int, 3>{});
  };

  // ---- main loop ------------------------------------------------------------------------
  // Stage k lives in buffer (k - kbeg) % 3.  Each wave waits for its own loads of stage k
  // (those of stage k+1 stay in flight) and for its own LDS reads of stage k-1; the
  // barrier then publishes stage k and frees stage k-1's buffer, which receives stage
  // k+2.  Every stage issues one stage's loads: past the end the last stage again
  // (harmless, never read), so the count in flight is the same at every wait and the
  // loop body has no branches.
  auto stage = [&](int kk, const uint8_t* cur, uint8_t* dst) {
    wait_cnt<D::NDW, 0>();
    __builtin_amdgcn_s_barrier();
    issue(kk + 2 < kend ? kk + 2 : kend - 1, dst);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      Frag F;
      load(cur, u, F);
      if constexpr (DEBUG) {
        v8i bf[TJ];
        expand(F, bf);
        const int64_t g = (int64_t)kk * 2 + u;
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
          for (int j = 0; j < TJ; ++j) {
            const v16f p = gs(F, bf, i, j);
            const int64_t c = n0 + wn + j * 32 + l32 - dbg.n0;
#pragma unroll
            for (int a = 0; a < 16; ++a) {
              const int64_t r = m0 + wm + i * 32 + 8 * (a >> 2) + 4 * kh + (a & 3) - dbg.m0;
              if (r >= 0 && r < dbg.mt && c >= 0 && c < dbg.nt) dbg.out[(g * dbg.mt + r) * dbg.nt + c] = (int32_t)p[a];
            }
          }
      } else if constexpr (FMT == 0) {
        v8i bf[TJ];
        expand(F, bf);
        // two tiles in flight: tile t+1's MFMAs are issued ahead of tile t's rescale
        constexpr int NTL = TI * TJ;
        v16f c[2], p[2];
        c[0] = sc(F, 0, 0);
        p[0] = gs(F, bf, 0, 0);
#pragma unroll
        for (int t = 0; t < NTL; ++t) {
          if (t + 1 < NTL) {
            c[(t + 1) & 1] = sc(F, (t + 1) / TJ, (t + 1) % TJ);
            p[(t + 1) & 1] = gs(F, bf, (t + 1) / TJ, (t + 1) % TJ);
          }
          epi(t / TJ, t % TJ, p[t & 1], c[t & 1]);
        }
      } else if constexpr (FMT == 2) {
        mma_nv(F);
      } else {
        mma4(F);
      }
    }
  };
  const int nk = kend - kbeg;
  int k = kbeg;
  // ---- low-rank up projection first: acc = lora_act[rows, :] L2[:, cols] ----------------
  // It depends on nothing of the main loop.  The operands of its first two k steps are
  // loaded before the first two stages' panels, so the MFMAs wait only for their own
  // loads while the panels stay in flight (loaded after the panels, they would wait
  // for those too: a wave's loads complete in issue order).
  // v_mfma_f32_32x32x16_bf16 on lora_act's bf16 hi/lo pairs and L2f, both in fragment
  // order: for a block of 32 rows (columns) and a k step of 16, the 64 lanes' operands
  // are 1 KB contiguous (lora_act: hi, then lo), so every load reads whole lines.  The
  // range covers whole 32-row blocks; rows past M hold whatever the workspace held
  // (their outputs are not stored), columns past N are zero.
  const bool lora = !DEBUG && rank > 0 && part <= 0;  // once per tile: whole, or the first part
  // NVFP4 scales the 4-bit sum by S_X S_W after the main loop, so its low-rank term comes
  // after that
  const bool lora_pre = lora && FMT != 2;
  const int R16 = (rank + 15) & ~15;
  const __amdgpu_buffer_rsrc_t rL = make_rsrc(lora_act + m0 * 2 * R16, (uint32_t)(((rowsA + 31) & ~31) * R16 * 4));
  const __amdgpu_buffer_rsrc_t rU = make_rsrc(L2 + n0 * R16, (uint32_t)(((rowsB + 31) & ~31) * R16 * 2));
  auto lora_load = [&](int s, v8bf (&b)[TJ], v8bf (&a)[TI][2]) {
#pragma unroll
    for (int j = 0; j < TJ; ++j)
      b[j] = __builtin_bit_cast(v8bf, buf_load16(rU, (uint32_t)(((((wn >> 5) + j) * (R16 >> 4) + s) * 64 + lane) * 16)));
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const uint32_t o = (uint32_t)(((((wm >> 5) + i) * (R16 >> 4) + s) * 2 * 64 + lane) * 16);
      a[i][0] = __builtin_bit_cast(v8bf, buf_load16(rL, o));
      a[i][1] = __builtin_bit_cast(v8bf, buf_load16(rL, o + 64 * 16));
    }
  };
  auto lora_mma = [&](const v8bf (&b)[TJ], const v8bf (&a)[TI][2]) {
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i][0], b[j], acc[i][j], 0, 0, 0);
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i][1], b[j], acc[i][j], 0, 0, 0);
      }
  };
  v8bf pb0[TJ], pa0[TI][2], pb1[TJ], pa1[TI][2];
  if (lora_pre) {
    lora_load(0, pb0, pa0);
    if (R16 > 16) lora_load(1, pb1, pa1);
  }
  issue(kbeg, lds0);
  issue(kbeg + 1 < kend ? kbeg + 1 : kend - 1, lds1);
  if (lora_pre) {
    lora_mma(pb0, pa0);
    if (R16 > 16) lora_mma(pb1, pa1);
    for (int s = 2; s < (R16 >> 4); ++s) {
      v8bf b[TJ], a[TI][2];
      lora_load(s, b, a);
      lora_mma(b, a);
    }
  }

  for (; k + 3 <= kend; k += 3) {
    stage(k, lds0, lds2);
    stage(k + 1, lds1, lds0);
    stage(k + 2, lds2, lds1);
  }
  if (nk % 3 >= 1) stage(k, lds0, lds2);
  if (nk % 3 == 2) stage(k + 1, lds1, lds0);
  wait_cnt<0, 0>();
  if constexpr (DEBUG) return;
  if constexpr (CHAIN) {
    chain_epilogue(acc, ch, M, N, m0, n0, rowsA, lds0, lds1, wave, lane, wn, l32, kh, Mp);
    return;
  }
  if constexpr (FMT == 2) {
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int a = 0; a < 16; ++a) acc[i][j][a] *= sxw;
    if (lora)
      for (int s = 0; s < (R16 >> 4); ++s) {
        v8bf b[TJ], a[TI][2];
        lora_load(s, b, a);
        lora_mma(b, a);
      }
  }

  // ---- store (or the partial tile) ------------------------------------------------------
  if (part < 0) {
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j) store_sub(acc[i][j], Y, ldy, ydtype, m0, n0, rowsA, N, wm + i * 32, wn + j * 32, l32, kh);
  } else {
    float* P = sch.partials + (size_t)(blockIdx.x - sch.full) * SH::PART;
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int a = 0; a < 16; ++a) P[((((wm >> 5) + i) * SH::CB + (wn >> 5) + j) * 16 + a) * 64 + lane] = acc[i][j][a];
  }
}

// Sum of the `split` partial tiles of one remaining tile, in part order (the result does
// not depend on which part finished first), stored like a whole tile.  One 64-thread
// block per 32 x 32 sub-tile: blockIdx.x = remaining tile * sub-tiles + sub-tile index,
// sub-tile = row block * CB + column block.
template <int TBM, int TBN>
__global__ __launch_bounds__(64) void k2_fixup(const float* __restrict__ partials, K2Sched sch, int64_t M,
                                               int64_t N, void* __restrict__ Y, int64_t ldy, int ydtype) {
  constexpr int CB = TBN / 32, NSUB = (TBM / 32) * CB, PF = NSUB * 16 * 64;
  const int lane = threadIdx.x;
  const uint32_t r = blockIdx.x / NSUB, sub = blockIdx.x % NSUB;
  const uint32_t t = sch.full + r;
  const int64_t m0 = (int64_t)(t / sch.tiles_n) * TBM, n0 = (int64_t)(t % sch.tiles_n) * TBN;
  const float* P = partials + (size_t)r * sch.split * PF + (size_t)sub * 16 * 64 + lane;
  v16f acc;
#pragma unroll
  for (int a = 0; a < 16; ++a) acc[a] = P[a * 64];
  for (uint32_t p = 1; p < sch.split; ++p) {
    const float* Q = P + (size_t)p * PF;
#pragma unroll
    for (int a = 0; a < 16; ++a) acc[a] += Q[a * 64];
  }
  const int64_t rowsA = M - m0 < TBM ? M - m0 : TBM;
  store_sub(acc, Y, ldy, ydtype, m0, n0, rowsA, N, (int)(sub / CB) * 32, (int)(sub % CB) * 32, lane & 31, lane >> 5);
}

// Sum of the chained epilogue's per-column-tile partials of the down projection, stored
// in the MMA form of lora_act (bf16 hi / lo pairs in fragment order) for fc2's kernel 2.
// A block takes 64 (token, rank column) elements; wave w sums the tiles w, w + 4, ... of
// each (64 consecutive floats per load), and wave 0 adds the four slices in wave order, so
// the result does not depend on which tile or block finished first.
__global__ __launch_bounds__(256) void k2_lora_reduce(const float* __restrict__ part, int ntiles, int64_t M, int R16,
                                                      uint16_t* __restrict__ la) {
  __shared__ float red[4][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t total = M * R16;
  const int64_t idx = (int64_t)blockIdx.x * 64 + lane;
  float v = 0.f;
  if (idx < total) {
#pragma unroll 4
    for (int t = w; t < ntiles; t += 4) v += part[(int64_t)t * total + idx];
  }
  red[w][lane] = v;
  __syncthreads();
  if (w == 0 && idx < total) {
    const float sum = ((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane];
    const int64_t m = idx / R16;
    store_lora_mma(la, m, (int)(idx - m * R16), R16 >> 4, sum);
  }
}

}  // namespace

// Sub-steps per stage: the largest of 2, 1 that divides K / 64.
static int sub_of(int64_t K) { return (K >> 6) % 2 == 0 ? 2 : 1; }

template <int FMT, int SUB>
static void launch_k2_t(const KernelLayer& L, int64_t M, const uint8_t* qX, const void* sX,
                        const void* lora_act, void* Y, int64_t ldy, int ydtype, const K2Sched& sch,
                        uint32_t nblocks, hipStream_t st) {
  hipLaunchKernelGGL((k2_gemm<FMT, false, SUB>), dim3(nblocks), dim3(NTHREADS), 0, st, qX, sX, M, L.qW,
                     L.sW, L.N, L.K, lora_act, L.L2f, L.rank, Y, ldy, ydtype, (int64_t)0, (int64_t)0, M, L.N, sch,
                     (int32_t*)nullptr);
}

template <int FMT, int SUB>
static int blocks_per_cu() {
  static int n = 0;  // per kernel instance; the same on every MI355X device
  if (n == 0) {
    int v = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, k2_gemm<FMT, false, SUB>, NTHREADS, 0) != hipSuccess ||
        v < 1)
      v = 1;
    n = v;
  }
  return n;
}

template <int FMT>
static int stream_blocks_per_cu() {
  static int n = 0;
  if (n == 0) {
    int v = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, k2_stream<FMT>, SShape<FMT>::NT, 0) != hipSuccess || v < 1)
      v = 1;
    n = v;
  }
  return n;
}

static int blocks_per_cu(int fmt, bool mma, int sub) {
  if (mma) return fmt == 0 ? stream_blocks_per_cu<0>() : (fmt == 2 ? stream_blocks_per_cu<2>() : stream_blocks_per_cu<1>());
  if (fmt == 0) return sub == 2 ? blocks_per_cu<0, 2>() : blocks_per_cu<0, 1>();
  return sub == 2 ? blocks_per_cu<1, 2>() : blocks_per_cu<1, 1>();
}

// Output tile of the kernel-2 variant for (format, activation form), and its partial
// tile size in floats.
static void tile_of(int fmt, bool mma, int& tbm, int& tbn, size_t& part) {
  if (mma && fmt == 0) { tbm = SShape<0>::BM; tbn = SShape<0>::BN; part = SShape<0>::PART; }
  else if (mma && fmt == 2) { tbm = SShape<2>::BM; tbn = SShape<2>::BN; part = SShape<2>::PART; }
  else if (mma) { tbm = SShape<1>::BM; tbn = SShape<1>::BN; part = SShape<1>::PART; }
  else { tbm = BM; tbn = BN; part = PART_FLOATS; }
}

K2Plan plan_k2(const KernelLayer& L, int64_t M, bool mma) {
  K2Plan p{};
  int tbm, tbn;
  size_t part;
  tile_of(L.fmt, mma, tbm, tbn, part);
  p.tiles_m = (uint32_t)((M + tbm - 1) / tbm);
  p.tiles_n = (uint32_t)((L.N + tbn - 1) / tbn);
  const uint32_t T = p.tiles_m * p.tiles_n;
  p.full = T;
  p.split = 1;
  p.bytes = 0;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    return p;
  const int sub = mma ? 2 : sub_of(L.K);
  const uint32_t G = (uint32_t)cus * (uint32_t)blocks_per_cu(L.fmt, mma, sub);  // blocks resident at once
  const uint32_t R = T % G;  // tiles of the last, partly filled round
  const uint32_t nst = (uint32_t)(L.K >> 6) / (uint32_t)sub;  // stages
  uint32_t S = R ? G / R : 1;
  if (S * 4 > nst * sub) S = nst * sub / 4;  // parts of at least 4 sub-steps
  if (S > nst) S = nst;
  // At most 4 parts: the partial tiles are written and read back by the fixup, and beyond
  // 4 parts that traffic costs more than the idle slots of the tail round it recovers
  // (measured on the QKV and batch-2 layers: 2-4 parts 3-6 us faster than 16).
  if (S > 4) S = 4;
  if (R == 0 || S < 2) return p;
  p.full = T - R;
  p.split = S;
  p.bytes = (size_t)R * S * part * sizeof(float);
  return p;
}

hipError_t launch_k2(const KernelLayer& L, int64_t M, const uint8_t* qX, const void* sX,
                     const void* lora_act, void* Y, int64_t ldy, int ydtype, bool mma,
                     void* workspace, size_t ws_bytes, hipStream_t st) {
  K2Plan p = plan_k2(L, M, mma);
  if (!workspace || ws_bytes < p.bytes || p.split < 2) {  // no split: every tile whole
    p.full = p.tiles_m * p.tiles_n;
    p.split = 1;
  }
  const uint32_t T = p.tiles_m * p.tiles_n, rem = T - p.full;
  const K2Sched sch{p.tiles_n, p.full, p.split, static_cast<float*>(workspace)};
  const uint32_t nblocks = p.full + rem * p.split;
#define K2_LAUNCH(F, SB) launch_k2_t<F, SB>(L, M, qX, sX, lora_act, Y, ldy, ydtype, sch, nblocks, st)
#define K2_STREAM(F)                                                                                        \
  hipLaunchKernelGGL((k2_stream<F>), dim3(nblocks), dim3(SShape<F>::NT), 0, st, qX, static_cast<const uint8_t*>(sX), M, \
                     L.qW, static_cast<const uint8_t*>(L.sW), L.N, L.K, static_cast<const uint16_t*>(lora_act),   \
                     L.L2f, L.rank, Y, ldy, ydtype, sch, K2Debug{}, L.tscale_x * L.tscale_w, K2Chain{})
  const int sub = sub_of(L.K);
  if (mma) {  // the activation side in MMA form: streamed kernel (K % 128 == 0: two sub-steps per stage)
    if (L.fmt == 0) K2_STREAM(0);
    else if (L.fmt == 2) K2_STREAM(2);
    else K2_STREAM(1);
  } else if (L.fmt == 0) {
    if (sub == 2) K2_LAUNCH(0, 2);
    else K2_LAUNCH(0, 1);
  } else {
    if (sub == 2) K2_LAUNCH(1, 2);
    else K2_LAUNCH(1, 1);
  }
#undef K2_LAUNCH
#undef K2_STREAM
  if (rem > 0) {
    const float* part = static_cast<const float*>(workspace);
    if (mma && L.fmt == 0)
      hipLaunchKernelGGL((k2_fixup<SShape<0>::BM, SShape<0>::BN>), dim3(rem * (SShape<0>::PART / 1024)), dim3(64), 0,
                         st, part, sch, M, L.N, Y, ldy, ydtype);
    else if (mma && L.fmt == 2)
      hipLaunchKernelGGL((k2_fixup<SShape<2>::BM, SShape<2>::BN>), dim3(rem * (SShape<2>::PART / 1024)), dim3(64), 0,
                         st, part, sch, M, L.N, Y, ldy, ydtype);
    else if (mma)
      hipLaunchKernelGGL((k2_fixup<SShape<1>::BM, SShape<1>::BN>), dim3(rem * (SShape<1>::PART / 1024)), dim3(64), 0,
                         st, part, sch, M, L.N, Y, ldy, ydtype);
    else
      hipLaunchKernelGGL((k2_fixup<BM, BN>), dim3(rem * 16), dim3(64), 0, st, part, sch, M, L.N, Y, ldy, ydtype);
  }
  return hipGetLastError();
}

hipError_t launch_k2_chain(const KernelLayer& L1, const KernelLayer& L2, int64_t M, const uint8_t* qX, const void* sX,
                           const void* lora_act, uint8_t* qX2, void* sX2, float* part, uint16_t* hidden, int64_t ldh,
                           hipStream_t st) {
  // whole tiles only (the epilogue needs the finished tile): no K split
  const uint32_t tiles_m = (uint32_t)((M + SShape<0>::BM - 1) / SShape<0>::BM);
  const uint32_t tiles_n = (uint32_t)(L1.N / SShape<0>::BN);
  const K2Sched sch{tiles_n, tiles_m * tiles_n, 1, nullptr};
  const K2Chain ch{qX2, static_cast<uint16_t*>(sX2), part, L2.inv_s, L2.L1f, (L2.rank + 15) / 16, hidden, ldh};
  hipLaunchKernelGGL((k2_stream<0, false, true>), dim3(tiles_m * tiles_n), dim3(SShape<0>::NT), 0, st, qX,
                     static_cast<const uint8_t*>(sX), M, L1.qW, static_cast<const uint8_t*>(L1.sW), L1.N, L1.K,
                     static_cast<const uint16_t*>(lora_act), L1.L2f, L1.rank, (void*)nullptr, (int64_t)0, 0, sch,
                     K2Debug{}, 1.0f, ch);
  return hipGetLastError();
}

hipError_t launch_lora_reduce(const KernelLayer& L1, const KernelLayer& L2, int64_t M, const float* part, void* la2,
                              hipStream_t st) {
  const int R16 = (L2.rank + 15) / 16 * 16;
  if (R16 == 0 || M == 0) return hipSuccess;
  const int64_t n = M * R16;
  hipLaunchKernelGGL(k2_lora_reduce, dim3((unsigned)((n + 63) / 64)), dim3(256), 0, st, part,
                     (int)(L1.N / SShape<0>::BN), M, R16, static_cast<uint16_t*>(la2));
  return hipGetLastError();
}

hipError_t launch_k2_debug(const KernelLayer& L, int64_t M, const uint8_t* qX, bool mma, int64_t m0,
                           int64_t n0, int64_t mt, int64_t nt, int32_t* out, hipStream_t st) {
  if (mma) {
    // the forward's streamed kernel on its own schedule (the same K split of the tail
    // round as the forward): every group of every window element is stored by exactly
    // one block, so no fixup runs
    K2Plan p = plan_k2(L, M, true);
    const uint32_t T = p.tiles_m * p.tiles_n, rem = T - p.full;
    const K2Sched sch{p.tiles_n, p.full, p.split, nullptr};
    hipLaunchKernelGGL((k2_stream<0, true>), dim3(p.full + rem * p.split), dim3(SShape<0>::NT), 0, st, qX,
                       (const uint8_t*)nullptr, M, L.qW, (const uint8_t*)nullptr, L.N, L.K, (const uint16_t*)nullptr,
                       (const uint16_t*)nullptr, 0, (void*)nullptr, (int64_t)0, 0, sch, K2Debug{out, m0, n0, mt, nt}, 1.0f,
                       K2Chain{});
    return hipGetLastError();
  }
  const uint32_t tn = (uint32_t)((nt + BN - 1) / BN), tm = (uint32_t)((mt + BM - 1) / BM);
  const K2Sched sch{tn, tm * tn, 1, nullptr};
  hipLaunchKernelGGL((k2_gemm<0, true, 1>), dim3(tm * tn), dim3(NTHREADS), 0, st, qX, (const void*)nullptr, M,
                     L.qW, (const void*)nullptr, L.N, L.K, (const void*)nullptr, (const uint16_t*)nullptr, 0,
                     (void*)nullptr, (int64_t)0, 0, m0, n0, m0 + mt, n0 + nt, sch, out);
  return hipGetLastError();
}

}  // namespace svdq
