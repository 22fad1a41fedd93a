// Kernel 4: the 4-bit weight-only layer (W4A16), the baseline the 4-bit activation path
// is set against.
//
// Method: Y = X Wd with Wd[k][n] = bf16(s_W[k / 64][n] q_W[n][k]): the weights are stored
// as INT4 codes with fp16 group scales and upcast to the activations' 16-bit type before
// a 16-bit product (jeonghoonpark.com "SVDQuant" review, section 3 "Quantization
// Preliminary": with unequal bit widths the narrower operand is upcast, so the product
// runs at 16-bit speed; the chatpaper.ai SVDQuant abstract measures the method's speed-up
// over a 4-bit weight-only baseline).  The weights use the layer's own INT4 quantizer
// (svdq_quantize_weights on W), in its storage form: codes [N][K/2], sign-magnitude
// nibbles with code 2j in the low nibble of byte j; fp16 scales [K/64][N].
//
// Design (gfx950): a dense bf16 contraction on v_mfma_f32_32x32x16_bf16, so the bound is
// the bf16 matrix-core peak.  A block of 8 waves owns a 256 x 256 tile of Y (wave w the
// 128 x 64 part at rows 128 (w >> 2), columns 64 (w & 3), as 4 x 2 accumulators: per 16-k
// step six 1 KB operand reads feed eight MFMAs) and walks K in stages of one group (64):
//  * X (256 rows x 128 bytes) goes global -> LDS by LDS-destination buffer loads, one
//    stage ahead, 16-byte slots XOR-swizzled by row so the operand reads of 16
//    consecutive rows fall in distinct bank groups;
//  * the weight codes of a stage (256 columns x 32 bytes) go global -> LDS the same way,
//    two stages ahead, and each lane's scale into a register; each lane upcasts 32 codes
//    of one column once per block (not once per wave): nibbles -> FP8 E4M3 subnormals
//    q 2^-9 -> fp32 (exact) -> times 2^9 s (exact: q s has at most 14 significant bits)
//    -> bf16, round to nearest even (the hardware conversion) -> the stage's LDS tile;
//  * two LDS buffers of 64 KB, one barrier per stage: it publishes stage k and frees the
//    other buffer for stage k+1's loads and upcast.
// Rows past M read as zeros and are not stored; columns past N have zero codes (their
// loads fall outside the range) and are not stored.
#include "common.hpp"
#include "kernels.hpp"

namespace svdq {
namespace {

constexpr int W16_BM = 256, W16_BN = 256, W16_WAVES = 8, W16_NT = 64 * W16_WAVES;
constexpr int W16_TI = 4, W16_TJ = 2;  // 32 x 32 accumulators per wave (128 x 64)
constexpr int W16_XB = W16_BM * 128;  // X bytes of a stage: 64 bf16 per row
constexpr int W16_WB = W16_BN * 128;  // upcast weight bytes of a stage
constexpr int W16_NDMA = W16_XB / 1024 / W16_WAVES;  // 1 KB X loads per wave and stage
// codes of a stage: 32 bytes per column
constexpr int W16_CB = W16_BN * 32;
static_assert(W16_CB == W16_WAVES * 1024, "one 1 KB code load per wave and stage");

// 16-byte slot of a 128-byte row, XOR-swizzled: the 16 rows of one 16-lane pass of a
// ds_read_b128 (same logical slot) land in 16 distinct 16-byte bank groups of 256 bytes
__device__ __forceinline__ int swz8(int row) { return (row ^ (row >> 3)) & 7; }

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}

// s_waitcnt vmcnt(N) lgkmcnt(0)
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "counter range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

__device__ __forceinline__ uint32_t bf16x2(float a, float b) {
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  const b2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Eight codes of one dword (code 2j in the low nibble of byte j) times sc = 2^9 s ->
// four bf16 pairs in code order
__device__ __forceinline__ uint4 upcast8(uint32_t d, float sc) {
  const uint32_t lo = (d & 0x07070707u) | ((d & 0x08080808u) << 4);  // codes 0, 2, 4, 6
  const uint32_t hi = ((d >> 4) & 0x07070707u) | (d & 0x80808080u);  // codes 1, 3, 5, 7
  const v2f a = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, false);      // 0, 2
  const v2f b = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, true);       // 4, 6
  const v2f c = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, false);      // 1, 3
  const v2f e = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, true);       // 5, 7
  return make_uint4(bf16x2(a.x * sc, c.x * sc), bf16x2(a.y * sc, c.y * sc), bf16x2(b.x * sc, e.x * sc),
                    bf16x2(b.y * sc, e.y * sc));
}

__device__ __forceinline__ void store_tile(const v16f& acc, void* Y, int64_t ldy, int ydtype, int64_t m0, int64_t n0,
                                           int64_t rows, int64_t N, int r_off, int c_off, int l32, int kh) {
  if (n0 + c_off + l32 >= N) return;
  const uint32_t ysz = ydtype == 0 ? 4u : 2u;
  const uint32_t ystep = (uint32_t)ldy * ysz;
  // base: element (m0, n0); range: to the end of row m0 + rows - 1 (rows past it dropped)
  const __amdgpu_buffer_rsrc_t rY =
      make_rsrc(static_cast<uint8_t*>(Y) + (m0 * ldy + n0) * ysz, (uint32_t)rows * ystep - (uint32_t)n0 * ysz);
  const uint32_t o = (uint32_t)(r_off + 4 * kh) * ystep + (uint32_t)(c_off + l32) * ysz;
#pragma unroll
  for (int a = 0; a < 16; ++a) {
    const uint32_t off = o + (uint32_t)(8 * (a >> 2) + (a & 3)) * ystep;
    if (ydtype == 0) buf_store4(__float_as_uint(acc[a]), rY, off);
    else buf_store2((uint16_t)f32_to_bf16_rne(acc[a]), rY, off);
  }
}

__global__ __launch_bounds__(W16_NT, 1) __attribute__((amdgpu_waves_per_eu(2, 2))) void k4_w4a16(
    const uint16_t* __restrict__ X, int64_t ldx, int64_t M, int64_t K, const uint8_t* __restrict__ qW,
    const uint16_t* __restrict__ sW, int64_t N, void* __restrict__ Y, int64_t ldy, int ydtype, uint32_t tiles_n) {
  // separate arrays for X and the upcast weights of each buffer, addressed statically
  // (the stage loop is unrolled by 2): the compiler then knows that the upcast's LDS
  // stores do not touch the X tile whose loads are in flight, and does not wait for them
  __shared__ __attribute__((aligned(1024))) uint8_t lx0[W16_XB];
  __shared__ __attribute__((aligned(1024))) uint8_t lx1[W16_XB];
  __shared__ __attribute__((aligned(1024))) uint8_t lw0[W16_WB];
  __shared__ __attribute__((aligned(1024))) uint8_t lw1[W16_WB];
  __shared__ __attribute__((aligned(1024))) uint8_t lc0[W16_CB];
  __shared__ __attribute__((aligned(1024))) uint8_t lc1[W16_CB];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, kh = lane >> 5;
  const int wr = (wave >> 2) * (32 * W16_TI), wc = (wave & 3) * (32 * W16_TJ);
  const int64_t m0 = (int64_t)(blockIdx.x / tiles_n) * W16_BM;
  const int64_t n0 = (int64_t)(blockIdx.x % tiles_n) * W16_BN;
  const int64_t rows = M - m0 < W16_BM ? M - m0 : W16_BM;
  const int64_t cols = N - n0 < W16_BN ? N - n0 : W16_BN;
  const int nst = (int)(K >> 6);

  // X: range to the end of the last valid row's K values; a row past it starts beyond
  // the range (ldx >= K), so its loads read zeros
  const __amdgpu_buffer_rsrc_t rX = make_rsrc(X + m0 * ldx, (uint32_t)((rows - 1) * ldx + K) * 2);
  uint32_t vx[W16_NDMA];
#pragma unroll
  for (int q = 0; q < W16_NDMA; ++q) {
    const int row = (wave + W16_WAVES * q) * 8 + (lane >> 3);
    vx[q] = (uint32_t)row * (uint32_t)ldx * 2 + (uint32_t)(((lane & 7) ^ swz8(row)) * 16);
  }
  auto issue_x = [&](int k, uint8_t* buf) {
#pragma unroll
    for (int q = 0; q < W16_NDMA; ++q) dma16(rX, buf + (wave + W16_WAVES * q) * 1024, vx[q], (uint32_t)k * 128);
  };

  // weights: lane t loads and upcasts column c = t >> 1, codes 32 h .. 32 h + 31 (h = t & 1)
  // of the stage's group; columns past N read zeros (codes) and get scale 0
  const int wcol = tid >> 1, wh = tid & 1;
  const bool col_ok = wcol < cols;
  const uint32_t kb = (uint32_t)(K >> 1);
  const __amdgpu_buffer_rsrc_t rQ = make_rsrc(qW + n0 * (int64_t)kb, (uint32_t)cols * kb);
  const __amdgpu_buffer_rsrc_t rS = make_rsrc(sW, (uint32_t)((K >> 6) * N * 2));
  const uint32_t qoff = (uint32_t)wcol * kb + (uint32_t)wh * 16;
  const uint32_t soff = (uint32_t)(n0 + wcol) * 2;
  // the scales ride in registers, one set per code buffer (a load of 2 bytes is range
  // checked on its own; the scale plane's size need not be a multiple of 4)
  uint32_t sw0, sw1;
  auto issue_codes = [&](int k, uint8_t* cbuf, uint32_t& sw) {
    dma16(rQ, cbuf + wave * 1024, qoff, (uint32_t)k * 32);
    sw = buf_load2(rS, soff + (uint32_t)k * (uint32_t)N * 2);
  };
  const int wsw = swz8(wcol);
  auto upcast = [&](const uint8_t* cbuf, uint32_t& sw, uint8_t* wbuf) {
    // pin the scale's use here (after the barrier that follows its arrival): left free,
    // the compiler moves the conversion up to the load and waits there for it
    asm volatile("" : "+v"(sw));
    const uint4 cw = *reinterpret_cast<const uint4*>(cbuf + tid * 16);
    const float s = col_ok ? (float)__builtin_bit_cast(_Float16, (uint16_t)sw) : 0.0f;
    const float sc = s * 512.0f;
    uint8_t* w = wbuf + wcol * 128;
    *reinterpret_cast<uint4*>(w + ((4 * wh + 0) ^ wsw) * 16) = upcast8(cw.x, sc);
    *reinterpret_cast<uint4*>(w + ((4 * wh + 1) ^ wsw) * 16) = upcast8(cw.y, sc);
    *reinterpret_cast<uint4*>(w + ((4 * wh + 2) ^ wsw) * 16) = upcast8(cw.z, sc);
    *reinterpret_cast<uint4*>(w + ((4 * wh + 3) ^ wsw) * 16) = upcast8(cw.w, sc);
  };

  v16f acc[W16_TI][W16_TJ];
#pragma unroll
  for (int i = 0; i < W16_TI; ++i)
#pragma unroll
    for (int j = 0; j < W16_TJ; ++j) acc[i][j] = v16f{};

  // operand reads: A row (B column) r, 16-k step s, lane half kh -> logical slot 2 s + kh
  auto compute = [&](const uint8_t* xbuf, const uint8_t* wbuf) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      v8bf A[W16_TI], B[W16_TJ];
#pragma unroll
      for (int i = 0; i < W16_TI; ++i) {
        const int r = wr + 32 * i + l32;
        A[i] = *reinterpret_cast<const v8bf*>(xbuf + r * 128 + (((2 * s + kh) ^ swz8(r)) * 16));
      }
#pragma unroll
      for (int j = 0; j < W16_TJ; ++j) {
        const int c = wc + 32 * j + l32;
        B[j] = *reinterpret_cast<const v8bf*>(wbuf + c * 128 + (((2 * s + kh) ^ swz8(c)) * 16));
      }
#pragma unroll
      for (int i = 0; i < W16_TI; ++i)
#pragma unroll
        for (int j = 0; j < W16_TJ; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[i], B[j], acc[i][j], 0, 0, 0);
    }
  };

  // Stage k lives in buffer k % 2 (X and upcast weights); the codes of stage k sit in code
  // buffer k % 2 from stage k-2 on.  At the top of stage k every load has arrived (X of
  // stage k and the codes of stage k+1, both issued at the top of stage k-1) and this
  // wave's upcast of stage k is in LDS; the barrier publishes stage k and, since every
  // wave has finished stage k-1, frees the other X / weight buffer (for X and the upcast
  // of stage k+1) and code buffer k % 2 (for the codes of stage k+2).  Past the end the
  // last stage is loaded again into free buffers, so the loop body has no branches.
  auto stage = [&](int k, const uint8_t* xcur, const uint8_t* wcur, uint8_t* xnxt, uint8_t* wnxt,
                   const uint8_t* cnxt, uint32_t& swn, uint8_t* ccur, uint32_t& swc) {
    wait_vm_lgkm0<0>();
    __builtin_amdgcn_s_barrier();
    issue_x(k + 1 < nst ? k + 1 : nst - 1, xnxt);
    upcast(cnxt, swn, wnxt);  // stage k+1 (or the last stage again)
    issue_codes(k + 2 < nst ? k + 2 : nst - 1, ccur, swc);
    compute(xcur, wcur);
  };

  issue_codes(0, lc0, sw0);
  issue_x(0, lx0);
  issue_codes(nst > 1 ? 1 : 0, lc1, sw1);
  wait_vm_lgkm0<0>();
  upcast(lc0, sw0, lw0);
  int k = 0;
  for (; k + 2 <= nst; k += 2) {
    stage(k, lx0, lw0, lx1, lw1, lc1, sw1, lc0, sw0);
    stage(k + 1, lx1, lw1, lx0, lw0, lc0, sw0, lc1, sw1);
  }
  if (k < nst) stage(k, lx0, lw0, lx1, lw1, lc1, sw1, lc0, sw0);
  wait_vm_lgkm0<0>();

#pragma unroll
  for (int i = 0; i < W16_TI; ++i)
#pragma unroll
    for (int j = 0; j < W16_TJ; ++j)
      store_tile(acc[i][j], Y, ldy, ydtype, m0, n0, rows, N, wr + 32 * i, wc + 32 * j, l32, kh);
}

}  // namespace

hipError_t launch_w4a16(int64_t M, int64_t K, int64_t N, const uint16_t* X, int64_t ldx, const uint8_t* qW,
                        const uint16_t* sW, void* Y, int64_t ldy, int ydtype, hipStream_t st) {
  const uint32_t tiles_m = (uint32_t)((M + W16_BM - 1) / W16_BM), tiles_n = (uint32_t)((N + W16_BN - 1) / W16_BN);
  hipLaunchKernelGGL(k4_w4a16, dim3(tiles_m * tiles_n), dim3(W16_NT), 0, st, X, ldx, M, K, qW, sW, N, Y, ldy, ydtype,
                     tiles_n);
  return hipGetLastError();
}

}  // namespace svdq
