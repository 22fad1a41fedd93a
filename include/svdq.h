/*
 * svdq.h - C ABI of the MI355X (gfx950) SVDQuant W4A4 + low-rank linear layer.
 *
 *   Y = Q(X diag(s)^-1) Q(R) + (X diag(s)^-1 L1) L2
 *
 * The layer equation and the split W_hat = L1 L2 + R (16-bit low-rank branch, 4-bit
 * residual) are those of the jeonghoonpark.com "SVDQuant" review, section 4.2, and of
 * the ch3chohch3.github.io post "从 Smooth Quant 到 SVD Quant", section "量化方案".
 * The two device entry points follow the two fused kernels of the review's section
 * 4.3 ("Nunchaku"): the low-rank down projection fused into activation quantization,
 * the low-rank up projection fused into the 4-bit GEMM.
 *
 * Conventions for every function below:
 *  - Row-major storage everywhere.  bf16 and fp16 values travel as uint16_t bit
 *    patterns.  Sizes are int64_t element counts.
 *  - "host" pointers are CPU memory; "device" pointers are GPU memory on the current
 *    HIP device.  The caller owns and allocates every buffer; the library allocates no
 *    device memory, keeps no global state besides a thread-local error message, and
 *    never synchronizes the device.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Device
 *    entry points only enqueue work on it and return; stream order is the only
 *    synchronization between them.
 *  - Every function returns an svdq_status; on failure svdq_last_error() describes
 *    it.  Nothing throws or aborts across this boundary.
 *
 * Formats (svdq_format):
 *  - SVDQ_INT4_G64: symmetric INT4, q in [-7, 7], one fp16 scale per 64 consecutive
 *    values along K, q = round-half-even(v / s), s = fp16(fp32(max|v| / 7)).  Codes
 *    are 4-bit sign-magnitude nibbles (bit 3 sign, bits 0-2 |q|).
 *  - SVDQ_MXFP4_G32: E2M1 codes (bit 3 sign, bits 0-2 index into
 *    {0, 0.5, 1, 1.5, 2, 3, 4, 6}) with one E8M0 byte (2^(byte - 127)) per 32 values,
 *    the exponent being the smallest e with 6 * 2^e >= max|v|; round half to even on
 *    the E2M1 grid, sign bit kept.
 *  - SVDQ_NVFP4_G16: the group-16, two-level-scale variant the ch3chohch3.github.io
 *    post discusses in its section "个人见解": E2M1 codes as above, one FP8 E4M3 scale
 *    per 16 values (bias 7, subnormals to 2^-9, largest finite 448) and one fp32 scale
 *    S per tensor, S = fp32(max|v| / 2688) (1 for an all-zero tensor).  Per group:
 *    s = E4M3(fp32(max|v| * fp32(1 / fp32(6 S)))) rounded half to even and saturating
 *    at 448; codes = E2M1 of fp32(v * fp32(1 / fp32(s S))), half to even, saturating at
 *    6, sign kept; a zero s gives sign-kept zero codes.  Value = S * s * e2m1(code).
 *    The weights' S comes from the residual, the activations' from the smoothed
 *    calibration statistic (fixed offline, like the smoothing factor).
 *  Two codes per byte: byte j of a row holds element 2j in the low nibble and
 *  element 2j+1 in the high nibble.  The quantizer formula is the review's section 3
 *  equation Q_X = round(X / s_X), s_X = max|X| / q_max (q_max 7 for INT4, 6 for FP4).
 */
#ifndef SVDQ_H
#define SVDQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SVDQ_OK = 0,
  SVDQ_EINVAL = 1,       /* bad argument: NULL pointer, size, alignment, range */
  SVDQ_EUNSUPPORTED = 2, /* valid but not supported (format, rank limit) */
  SVDQ_ENUMERIC = 3,     /* non-finite input where finite values are required */
  SVDQ_EHIP = 4          /* HIP runtime error reported at launch */
} svdq_status;

typedef enum { SVDQ_INT4_G64 = 0, SVDQ_MXFP4_G32 = 1, SVDQ_NVFP4_G16 = 2 } svdq_format;
/* Output types of kernel 2: fp32, bf16, or bf16 of GELU(y) (the exact GELU y Phi(y),
 * Phi the standard normal CDF, evaluated in fp32, then rounded once to bf16), the
 * activation between the two layers of an MLP pair. */
typedef enum { SVDQ_F32 = 0, SVDQ_BF16 = 1, SVDQ_BF16_GELU = 2 } svdq_dtype;

/* How kernel 1 hands the activation side to kernel 2 (both calls must agree).
 *   PACKED: the format's storage form: qX [M][K/2] 4-bit codes (INT4 sign-magnitude
 *           nibbles, MXFP4 E2M1), sX [K/G][M] fp16 bits (INT4) or E8M0 bytes (MXFP4),
 *           lora_act [M][R16] fp32.
 *   MMA:    the matrix-core operand form, which kernel 2 streams into LDS without
 *           converting.  Mp = M rounded up to a multiple of 4.
 *           INT4: qX [M][K] bytes, 64 per token and group: the codes as matrix-core
 *           FP6 E2M3 operands, 6-bit fields sign << 5 | |q| (exponent 0: value q / 8).
 *           Group half h (32 codes) is six 32-bit words w0..w5 holding field f at bit
 *           6 f of their 192-bit concatenation, field f carrying k = 32 h + 16 (f & 1)
 *           + (f >> 1) of the group; it is stored at byte 32 h as [w0 w1 w2 w3 w4 w5
 *           0 0]; sX [K/64][Mp] fp16 bits.
 *           MXFP4: the PACKED codes in token pairs: byte b of token m's code row at
 *           (m / 2) * K + (b / 64) * 128 + (m % 2) * 64 + b % 64 ((M rounded up to 2) *
 *           K/2 bytes); sX [K/32][Mp] E8M0 bytes.
 *           NVFP4: the codes in token pairs as for MXFP4, but inside each block of 64
 *           K values code k is at nibble 2 (16 ((k / 8) % 2) + 4 (k / 16)) + (k % 8) of the
 *           block's 32 bytes (the lane order of the bf16 matrix core: eight codes of one
 *           group of 16 per lane and K step); sX [K/64][Mp][4]: the four E4M3 group scales
 *           of a row and 64-block contiguous.
 *           Both: lora_act as bf16 pairs hi = bf16(v), lo = bf16(v - hi) of the fp32
 *           value v, in the matrix core's fragment order (each 16-byte load of kernel
 *           2 then reads whole lines): with S = R16 / 16, the hi (p = 0) and lo (p = 1)
 *           halves of value (m, j) at bf16 element
 *             ((((m / 32) S + j / 16) 2 + p) 64 + m % 32 + 32 ((j / 8) % 2)) 8 + j % 8,
 *           (M rounded up to 32) * R16 * 2 elements; the rows past M are not written. */
typedef enum { SVDQ_ACT_PACKED = 0, SVDQ_ACT_MMA = 1 } svdq_act_form;

#define SVDQ_MAX_RANK 128

/* Device-resident description of one packed layer (all pointers device memory,
 * owned by the caller, produced by svdq_pack_weights, then svdq_prepare_lowrank_down,
 * svdq_prepare_lowrank and svdq_prepare_weights for the kernels' layouts).
 * R16 below is rank rounded up to a multiple of 16.
 *   inv_s  [K]        fp32  reciprocal smoothing factor, fp32(1 / fp32(s))
 *   L1f    R16 * K    bf16  down projection in kernel 1's fragment order, as
 *                           svdq_prepare_lowrank_down writes it
 *   L2f    N32 * R16  bf16  up projection in kernel 2's fragment order, as
 *                           svdq_prepare_lowrank writes it (N32 = N rounded up to 32)
 *   qW                u8    residual codes along K per output channel, in the kernel
 *                           layout of svdq_prepare_weights (INT4: column pairs)
 *   sW                group-major scales as svdq_prepare_weights writes them: INT4
 *                           fp16, MXFP4 E8M0 bytes, rows padded to Np (16-byte aligned)
 * L1f/L2f may be NULL iff rank == 0. */
typedef struct svdq_layer {
  int64_t K, N;
  int32_t rank;
  int32_t fmt; /* svdq_format */
  const float* inv_s;
  const uint16_t* L1f;
  const uint16_t* L2f;
  const uint8_t* qW;
  const void* sW;
  /* NVFP4 only (host values, ignored otherwise): the weights' and the activations'
   * fp32 tensor scales, as svdq_pack_weights writes them after the group scales */
  float tscale_w, tscale_x;
} svdq_layer;

/* Thread-local description of the last failure in this thread ("" after success). */
const char* svdq_last_error(void);

/* ----------------------------------------------------------------- host side ---- */

/* Calibration statistic max over rows m of |X[m][k]| for each input channel k
 * (the max|X_j| of the smoothing-factor formula, ch3chohch3.github.io post, section
 * "Smooth Quant（W8A8）").  X: host bf16 [M][ldx]; out: host fp32 [K].
 * EINVAL on NULL / M < 1 / K < 1 / ldx < K. */
svdq_status svdq_act_absmax(int64_t M, int64_t K, const uint16_t* X, int64_t ldx, float* out);

/* Sizes in bytes of the packed residual buffers for a K x N layer.  NVFP4: sW holds the
 * E4M3 group scales [K/16][N] followed by two fp32 values, the weights' tensor scale and
 * the activations' tensor scale. */
svdq_status svdq_weight_sizes(int64_t K, int64_t N, int32_t fmt, size_t* qW_bytes,
                              size_t* sW_bytes);

/* Offline pack (host only, fp64 internally; multi-threaded).
 *   s_j = max(a_j,1e-5)^alpha / max(w_j,1e-5)^(1-alpha), w_j = max_n |W[j][n]|
 *     (ch3chohch3.github.io post, "Smooth Quant（W8A8）", smoothing-factor equation);
 *   W_hat = diag(fp32(s)) W;  truncated SVD W_hat ~ U_r Sigma_r V_r^T computed from the
 *     Gram matrix of W_hat with the library's own symmetric eigensolver;
 *   L1 = U_r Sigma_r, L2 = V_r^T, both rounded to bf16 (review, section 4.2);
 *   R = W_hat - L1 L2 with the rounded factors; R quantized per output column n in
 *     groups along K (format fmt).
 * Inputs: W host bf16 [K][N]; act_absmax host fp32 [K] or NULL for no smoothing
 * (s = 1); alpha in [0,1]; 0 <= rank <= min(K, N, SVDQ_MAX_RANK).
 * Outputs (host, caller-allocated): s_out, inv_s_out [K] fp32; L1t_out [rank][K] bf16
 * (L1 transposed: row j = sigma_j u_j); L2_out [rank][N] bf16; qW_out [N][K/2];
 * sW_out [K/G][N] (NVFP4: then the two fp32 tensor scales, the activations' taken from
 * max_k fp32(act_absmax[k] * inv_s[k]), 1 when act_absmax is NULL); R_out optional fp32
 * [K][N] (NULL to skip).
 * Errors: EINVAL (NULL, K % 128 != 0, N < 1, alpha out of range, bad rank),
 * ENUMERIC (non-finite W or act_absmax), EUNSUPPORTED (fmt). */
svdq_status svdq_pack_weights(int64_t K, int64_t N, const uint16_t* W, const float* act_absmax,
                              float alpha, int32_t rank, int32_t fmt, float* s_out,
                              float* inv_s_out, uint16_t* L1t_out, uint16_t* L2_out,
                              uint8_t* qW_out, void* sW_out, float* R_out);

/* Offline pack with iterative refinement of the split (jeonghoonpark.com "SVDQuant"
 * review, the discussion after "Limitation", item on accuracy: R optimised repeatedly
 * rather than taken from one split).  Iterate 0 is svdq_pack_weights' split; iterate
 * t = 1..iters takes the rank-r split of W_hat - deq(Q(R_{t-1})), rounds its factors to
 * bf16 and sets R_t = W_hat - L1 L2.  The outputs are those of the iterate with the
 * smallest E = ||W_hat - L1 L2 - deq(Q(R))||_F (Frobenius norm, fp64; the first on ties),
 * so the result is never worse than the plain split, and iters = 0 gives exactly
 * svdq_pack_weights' outputs.  err_out: optional host double [iters + 1], the E of every
 * iterate.  Each iterate costs about one plain pack.  Arguments, outputs and errors as
 * for svdq_pack_weights; EINVAL for iters outside [0, 64]. */
svdq_status svdq_pack_weights_refined(int64_t K, int64_t N, const uint16_t* W, const float* act_absmax,
                                      float alpha, int32_t rank, int32_t fmt, int32_t iters, float* s_out,
                                      float* inv_s_out, uint16_t* L1t_out, uint16_t* L2_out, uint8_t* qW_out,
                                      void* sW_out, float* R_out, double* err_out);

/* Quantize a given fp32 residual R [K][N] (host) per output column in groups along K:
 * the last step of svdq_pack_weights on its own.  Outputs as in svdq_pack_weights
 * (NVFP4: the activations' tensor scale is written as 1). */
svdq_status svdq_quantize_weights(int64_t K, int64_t N, const float* R, int32_t fmt,
                                  uint8_t* qW_out, void* sW_out);

/* Fold an off-the-shelf LoRA (X A B on unsmoothed X) into the low-rank branch without
 * touching the quantized residual (SVDQuant abstract, chatpaper.ai: adapters run
 * without re-quantization).  X A B = (X diag(s)^-1)(diag(s) A) B, so
 *   L1t_out = [L1t ; bf16(lora_scale * diag(s) A)^T]   ([rank+lr][K])
 *   L2_out  = [L2 ; B]                                  ([rank+lr][N])
 * Host pointers: s [K] fp32; L1t [rank][K]; L2 [rank][N]; A [K][lr]; B [lr][N] bf16.
 * EINVAL / EUNSUPPORTED when rank + lr exceeds SVDQ_MAX_RANK. */
svdq_status svdq_concat_lora(int64_t K, int64_t N, const float* s, int32_t rank,
                             const uint16_t* L1t, const uint16_t* L2, int32_t lora_rank,
                             const uint16_t* A, const uint16_t* B, float lora_scale,
                             uint16_t* L1t_out, uint16_t* L2_out);

/* Offline device layout of the down projection: L1^T [rank][K] (as svdq_pack_weights
 * writes it) reordered so that each 16-byte load of kernel 1 reads whole 128-byte lines.
 * With NT = R16 / 16, chunk c = k / 64, rank tile t = j / 16, lane l = (j % 16) +
 * 16 ((k % 64) / 16) and e = k % 16:
 *   L1f[((c NT + t) 64 + l) 16 + e] = L1t[j][k] (j < rank), 0 (rank <= j < R16),
 * i.e. for one chunk and rank tile, lane l's 16 consecutive channels of rank row j are
 * 32 contiguous bytes.  Host pointers; L1t [rank][K], L1f_out R16 * K bf16.  EINVAL on
 * bad sizes (K a positive multiple of 64) or NULL pointers (rank 0: nothing written). */
svdq_status svdq_prepare_lowrank_down(int64_t K, int32_t rank, const uint16_t* L1t, uint16_t* L1f_out);

/* Offline device layout of the up projection: L2 [rank][N] in the matrix core's
 * fragment order, so that each 16-byte load of kernel 2 reads whole lines.  With S =
 * R16 / 16:
 *   L2f[(((n / 32) S + j / 16) 64 + n % 32 + 32 ((j / 8) % 2)) 8 + j % 8] = L2[j][n]
 * for j < rank and n < N, and 0 for rank <= j < R16 or N <= n < N32 (N rounded up to
 * 32).  Host pointers; L2 [rank][N], L2f_out N32 * R16 bf16.  EINVAL on bad sizes or
 * NULL pointers (rank 0: nothing to write, pointers unused). */
svdq_status svdq_prepare_lowrank(int64_t N, int32_t rank, const uint16_t* L2, uint16_t* L2f_out);

/* Offline device layout of the residual weights (host pointers).  The values are those
 * of svdq_pack_weights / svdq_quantize_weights; only their encoding changes.  Np = N
 * rounded up to a multiple of 4; scale rows are padded to it.
 *   MXFP4: qW_out: the codes as stored, columns in pairs as for INT4 below ((N rounded
 *          up to 2) * K/2 bytes); sW_out [K/32][Np] E8M0 bytes (padding 127).
 *   INT4:  qW_out: (N rounded up to 2) * K/2 bytes.  Each 16 bytes of a column (32
 *          codes, a group half) become four words v0..v3 from which masks alone give
 *          the half's six FP6 operand words w0..w5 (fields and k order as in the MMA
 *          activation form below):
 *          with Z0 = the bits 3-4 of fields 0-4 (0x18618618) and Z1 = bits 1-2, 7-8,
 *          13-14, 19-20, 25-26 and 31 (0x86186186),
 *            v0 = w0 | (w2 & Z0), v1 = w1 | (w2 & Z1), v2 = w3 | (w5 & Z0),
 *            v3 = w4 | (w5 & Z1);
 *          w0 = v0 & ~Z0, w1 = v1 & ~Z1, w2 = (v0 & Z0) | (v1 & Z1) (w3..w5 likewise),
 *          since every field has zero exponent bits (bits 3-4).  Columns are stored
 *          in pairs: byte b of column n (in the order above) is at
 *          (n / 2) * K + (b / 64) * 128 + (n % 2) * 64 + b % 64, so the 64-byte
 *          segments of columns 2j and 2j+1 for 128 consecutive K share a 128-byte line;
 *          with N odd the last pair's second column is zero.
 *          sW_out: the fp16 scale bits [K/64][Np] ((K/64) * Np * 2 bytes), padding 0.
 *   NVFP4: qW_out: codes in column pairs as for MXFP4, each 64-block in the lane order
 *          of the MMA activation form below; sW_out [K/64][Np][4] E4M3 bytes (padding
 *          0).  The tensor scales are not copied: they go into svdq_layer. 
 * EINVAL on bad sizes, ENUMERIC on a negative or non-finite scale. */
svdq_status svdq_prepare_weights(int64_t K, int64_t N, int32_t fmt, const uint8_t* qW,
                                 const void* sW, uint8_t* qW_out, void* sW_out);

/* ---------------------------------------------------------------- device side ---- */

/* Kernel 1: smooth, quantize and down-project the activations in one pass over X
 * (review section 4.3: down projection fused with the quantization kernel, sharing
 * the activation read).
 *   X        device bf16 [M][ldx], 16-byte aligned rows (ldx % 8 == 0)
 *   form     svdq_act_form of the outputs:
 *   qX       device                       codes of X_hat = X diag(inv_s)
 *   sX       device                       their group scales
 *   lora_act device                       X_hat L1, columns >= rank written as zero
 *                                         (unused when rank == 0)
 * One launch (at rank 0, K >= 8192 and ceil(M / 16) <= 2 x CUs: the chunks of 64 along K
 * cut into 4 contiguous ranges, one block each, the same codes and scales).
 * M == 0 is a no-op.  EINVAL on NULL / misalignment / ldx < K; EUNSUPPORTED when
 * M * K >= 2^35 (the scale planes are addressed through 32-bit offsets); EHIP on launch
 * error. */
svdq_status svdq_quantize_act_lora_down(const svdq_layer* layer, int64_t M, const uint16_t* X,
                                        int64_t ldx, int32_t form, uint8_t* qX, void* sX,
                                        void* lora_act, void* stream);

/* Kernel 2: W4A4 GEMM on the codes with per-group rescaling by s_X s_W and the
 * low-rank up projection (lora_act L2) added in the epilogue (review section 4.3: up
 * projection fused with the 4-bit kernel).
 *   form, qX, sX, lora_act  as written by kernel 1 (device)
 *   Y                 device [M][ldy], svdq_dtype ydtype; ldy < 2^22 elements
 *                     (EUNSUPPORTED otherwise: a tile's rows are addressed through a
 *                     32-bit range)
 *   workspace         optional device scratch (NULL / ws_bytes 0: none), 256-byte
 *                     aligned.  With at least svdq_gemm_workspace_bytes bytes, the
 *                     output tiles that would form a last, partly filled round
 *                     of resident blocks are split along K, their fp32 partial tiles
 *                     kept there and added in a fixed order by a second kernel; the
 *                     result is deterministic for a given device and workspace choice.
 * Y is overwritten (no accumulation into existing contents). */
svdq_status svdq_gemm_w4a4_lora_up(const svdq_layer* layer, int64_t M, int32_t form,
                                   const uint8_t* qX, const void* sX, const void* lora_act,
                                   void* Y, int64_t ldy, int32_t ydtype, void* workspace,
                                   size_t ws_bytes, void* stream);

/* Workspace bytes kernel 2 uses for its split on the current device (0: no split). */
size_t svdq_gemm_workspace_bytes(const svdq_layer* layer, int64_t M, int32_t form);

/* Bytes of device workspace svdq_linear_forward needs for M rows on the current device:
 * the MMA-form qX, sX and lora_act, then one region for kernel 1's per-part sums (when
 * it is cut along K) and, after them, kernel 2's split workspace; each 256-byte
 * aligned. */
size_t svdq_workspace_bytes(const svdq_layer* layer, int64_t M);

/* The number of contiguous K ranges svdq_linear_forward cuts kernel 1's blocks of 16
 * tokens into for M rows on the current device (1: one pass), for callers that time or
 * reproduce the forward's launches.  At K >= 8192 with ceil(M / 16) <= 2 x CUs every block
 * is cut, into 4; at shorter K and rank 0, when the blocks leave a last round of one block
 * per CU at most half full, only that round's blocks are cut, into min(8, CUs / blocks in
 * it, K / 64) ranges (the FLUX.1 layers' 4608 tokens on 256 CUs: 32 blocks, 8 ranges).
 * Returns 0 for a NULL layer, bad dimensions or M < 0. */
int32_t svdq_forward_k1_parts(const svdq_layer* layer, int64_t M);

/* The public layer Y = Q(X diag(s)^-1) Q(R) + (X diag(s)^-1 L1) L2 (decomposition
 * equation of the jeonghoonpark.com "SVDQuant" review, section 4.2), computed the way
 * the review's section 4.3 ("Nunchaku", Figure 6(b)) fuses it: two kernels instead of
 * four, the down projection sharing the quantization kernel's read of X and the up
 * projection sharing the 4-bit GEMM's output tile.  Kernel 1 then kernel 2 on `stream`
 * with the activation side in MMA form, intermediates in `workspace` (device, >=
 * svdq_workspace_bytes, 256-byte aligned, caller-owned; its contents on entry do not
 * matter).  The same launches as the two calls above with form = SVDQ_ACT_MMA and
 * kernel 2 given its split workspace, and the results identical bit for bit, except at
 * K >= 8192 with rank > 0 and at most two 16-token blocks per compute unit
 * (ceil(M / 16) <= 2 x CUs): there kernel 1 runs cut into 4 contiguous ranges of its
 * 64-wide chunks, one block per range, and a second small kernel adds the ranges' fp32
 * down-projection sums in range order.  Codes and scales are the same; lora_act differs
 * from the one-pass kernel only in the order of its fp32 additions (deterministic).  (At
 * rank 0 kernel 1 has no sums to add, and svdq_quantize_act_lora_down takes the same
 * cut itself.)
 *   X  device bf16 [M][ldx] (16-byte aligned rows); Y device [M][ldy], svdq_dtype
 *   ydtype, overwritten; columns >= N of each Y row are not touched.
 * M == 0 is a no-op.  EINVAL on NULL / misalignment / small workspace; EUNSUPPORTED on
 * ldy >= 2^22; EHIP on launch error. */
svdq_status svdq_linear_forward(const svdq_layer* layer, int64_t M, const uint16_t* X,
                                int64_t ldx, void* Y, int64_t ldy, int32_t ydtype,
                                void* workspace, size_t ws_bytes, void* stream);

/* Size in bytes of the fixed device array svdq_linear_forward_noalloc uses as its
 * workspace (one per device): 64 MiB, enough for every FLUX.1 layer workload of this
 * library (the largest, the MLP fc2 layer at 4608 tokens, needs about 62 MB). */
#define SVDQ_NOALLOC_SCRATCH_BYTES (64u << 20)

/* For callers that cannot allocate device memory (code under HIP stream capture, serving
 * loops that must not call an allocator): svdq_linear_forward with its workspace in a
 * fixed device array of the library (SVDQ_NOALLOC_SCRATCH_BYTES, one copy per device,
 * held until the process ends) instead of a caller's buffer.  Same kernels, launches and
 * results, bit for bit, as svdq_linear_forward.  The call allocates nothing: on its first
 * call on a device it looks up that device's copy of the array (hipGetSymbolAddress).
 * The array needs no clearing: every byte a call reads is written earlier in that call.
 * Every call on one device shares that device's array, so calls that overlap on one
 * device (other streams or threads without ordering between them) race and must not be
 * made.  Arguments and errors as for svdq_linear_forward; EUNSUPPORTED, with nothing
 * launched, when svdq_workspace_bytes(layer, M) exceeds SVDQ_NOALLOC_SCRATCH_BYTES. */
svdq_status svdq_linear_forward_noalloc(const svdq_layer* layer, int64_t M, const uint16_t* X,
                                        int64_t ldx, void* Y, int64_t ldy, int32_t ydtype,
                                        void* stream);

/* The unfused baseline (jeonghoonpark.com "SVDQuant" review, section 4.3, Figure 6(a)):
 * the same layer with the low-rank branch run as kernels of its own, the arrangement
 * the fused path is measured against.  Four launches on `stream`: kernel 1 without the
 * down projection, a down-projection kernel that reads X a second time (lora_act into
 * the workspace), kernel 2 without the up projection (writes Q(X_hat) Q(R) to Y), and
 * an up-projection kernel that reads Y back and writes Y + lora_act L2.  Arguments,
 * workspace size (svdq_workspace_bytes) and errors as for svdq_linear_forward, except
 * that ydtype SVDQ_BF16_GELU is EUNSUPPORTED (the last kernel adds to Y).  The
 * codes and the 4-bit product are bit-identical to the fused path's; Y differs from it
 * only by the rounding of the intermediate Y (bf16 output: rounded twice) and the order
 * of the fp32 additions. */
svdq_status svdq_linear_forward_unfused(const svdq_layer* layer, int64_t M, const uint16_t* X,
                                        int64_t ldx, void* Y, int64_t ldy, int32_t ydtype,
                                        void* workspace, size_t ws_bytes, void* stream);

/* The 4-bit weight-only baseline (W4A16): the weights stored as 4-bit codes and upcast
 * to the activations' 16-bit type before a 16-bit product, the arrangement the method's
 * speed-up is measured against (jeonghoonpark.com "SVDQuant" review, section 3
 * "Quantization Preliminary", on operands of unequal bit width; chatpaper.ai SVDQuant
 * abstract, the 3.0x over a 4-bit weight-only baseline).
 *   Y[m][n] = sum_k X[m][k] Wd[k][n],  Wd[k][n] = bf16(sW[k/64][n] * q[n][k])
 * (the exact product of scale and code rounded once to bf16, nearest, ties to even),
 * accumulated in fp32 on the bf16 matrix core; no smoothing and no low-rank branch.
 *   X   device bf16 [M][ldx], 16-byte aligned, ldx % 8 == 0, ldx >= K
 *   qW  device INT4 codes of W in the storage form of svdq_quantize_weights / pack
 *       ([N][K/2], sign-magnitude nibbles, code 2j in the low nibble of byte j; make
 *       them with svdq_quantize_weights on W itself), 16-byte aligned
 *   sW  device fp16 scale bits [K/64][N]
 *   Y   device [M][ldy], fp32 (SVDQ_F32) or bf16 (SVDQ_BF16)
 * All buffers are the caller's; one launch on `stream`.  M == 0 is a no-op.  EINVAL on
 * NULL, misalignment, K not a positive multiple of 64, N < 1, ldx < K or ldy < N;
 * EUNSUPPORTED for another ydtype or ldx / ldy >= 2^22 or K/64 * N >= 2^31; EHIP on
 * launch error. */
svdq_status svdq_w4a16_gemm(int64_t M, int64_t K, int64_t N, const uint16_t* X, int64_t ldx,
                            const uint8_t* qW, const uint16_t* sW, void* Y, int64_t ldy,
                            int32_t ydtype, void* stream);

/* ---------------------------------------------------- the chained MLP pair ---- */
/* Two layers with GELU between them, Y = fc2(bf16(GELU(fc1(X)))), fc1.N == fc2.K.  The
 * fused-kernel design of the jeonghoonpark.com "SVDQuant" review (section 4.3,
 * "Nunchaku", Figure 6(b)) carried one step further, for the cost the ch3chohch3.github.io
 * post "从 Smooth Quant 到 SVD Quant" names in its "量化方案" section (16-bit activations
 * written and read back from HBM between kernels): fc1's kernel 2 runs fc2's kernel 1 on
 * its finished output tile, so the 16-bit hidden activation G never goes to memory.
 *   SVDQ_MLP_CHAINED: kernel 1 of fc1; fc1's kernel 2 with the chained epilogue (GELU,
 *     smoothing by fc2's 1 / s, fc2's INT4 codes and fp16 scales in MMA form, and the
 *     partial down projections by fc2's L1 over each 128-channel column tile); the
 *     partials summed in a fixed order into fc2's lora_act; fc2's kernel 2.  INT4
 *     layers only (EUNSUPPORTED otherwise).
 *   SVDQ_MLP_SEPARATE: the two layers as two svdq_linear_forward calls, fc1's with
 *     ydtype SVDQ_BF16_GELU into a bf16 G in the workspace (the baseline).
 * Both modes compute G the same way, and fc2's codes and scales from equal G are equal;
 * Y differs between them only by the fp32 summation order of fc2's down projection and
 * of fc1's K-split tiles (the chained fc1 computes every tile whole). */
typedef enum { SVDQ_MLP_CHAINED = 0, SVDQ_MLP_SEPARATE = 1 } svdq_mlp_mode;

/* Workspace bytes of svdq_mlp_forward for M tokens in `mode` on the current device (0 on
 * invalid arguments). */
size_t svdq_mlp_workspace_bytes(const svdq_layer* fc1, const svdq_layer* fc2, int64_t M, int32_t mode);

/* The pair on `stream`.  X device bf16 [M][ldx] (16-byte aligned rows); Y device
 * [M][ldy] (svdq_dtype ydtype), overwritten; workspace device, >= svdq_mlp_workspace_bytes,
 * 256-byte aligned, contents on entry irrelevant.  M == 0 is a no-op.  EINVAL on NULL /
 * misalignment / small workspace / fc1.N != fc2.K; EUNSUPPORTED on a chained non-INT4
 * pair or ldy >= 2^22; EHIP on launch error. */
svdq_status svdq_mlp_forward(const svdq_layer* fc1, const svdq_layer* fc2, int64_t M, const uint16_t* X,
                             int64_t ldx, void* Y, int64_t ldy, int32_t ydtype, int32_t mode, void* workspace,
                             size_t ws_bytes, void* stream);

/* The chained step alone: fc1's kernel 2 on fc1's MMA-form activation side (qX, sX,
 * lora_act from svdq_quantize_act_lora_down with SVDQ_ACT_MMA), every output tile whole,
 * with fc2's kernel 1 in its epilogue.  Writes (device):
 *   qX2       fc2's codes in MMA form, [M][K2] bytes (K2 = fc1.N = fc2.K), 16-byte aligned
 *   sX2       fc2's fp16 scales in MMA form, [K2/64][Mp] (Mp = M rounded up to 4)
 *   lora_part fp32 [K2/128][M][R16], R16 = fc2.rank rounded up to 16: the down
 *             projection of each token over each 128-channel column tile (unused when
 *             fc2.rank == 0)
 *   hidden    optional (NULL: not written): G = bf16(GELU(H)) [M][ldh], ldh >= K2, ldh a
 *             multiple of 8, 16-byte aligned
 * INT4 layers only.  Errors as for svdq_gemm_w4a4_lora_up. */
svdq_status svdq_mlp_chain_gemm(const svdq_layer* fc1, const svdq_layer* fc2, int64_t M, const uint8_t* qX,
                                const void* sX, const void* lora_act, uint8_t* qX2, void* sX2, float* lora_part,
                                uint16_t* hidden, int64_t ldh, void* stream);

/* fc2's lora_act in MMA form (the layout svdq_quantize_act_lora_down writes with
 * SVDQ_ACT_MMA, 16-byte aligned) = the sum of lora_part over the K2/128 column tiles, in
 * a fixed order (tiles t = s mod 4 summed in tile order for each s, then the four sums
 * in order of s), so the result is deterministic.  No-op when fc2.rank == 0 or M == 0. */
svdq_status svdq_mlp_chain_reduce(const svdq_layer* fc1, const svdq_layer* fc2, int64_t M, const float* lora_part,
                                  void* lora_act2, void* stream);

/* Diagnostic: the exact integer group sums I[g][m][n] = sum_{k in group g} qX[m][k]
 * qW[n][k] (INT4 only; the review's section 3 product Q_X Q_W, taken per group) for the
 * window rows [m0, m0+mt) x cols [n0, n0+nt).  out: device int32 [K/64][mt][nt].
 *   form = SVDQ_ACT_MMA: qX in kernel 1's MMA form; the kernel is the one
 *     svdq_linear_forward and svdq_gemm_w4a4_lora_up (MMA form) run, instantiated with
 *     an epilogue that stores each group's MFMA result instead of rescaling it: the same
 *     launch schedule (including the K split of the last round), loads, LDS layout,
 *     weight expansion and group-sum instruction.
 *   form = SVDQ_ACT_PACKED: qX packed [M][K/2]; the packed-form kernel 2's main loop.
 * Synchronous (waits for the stream) so it can be used from tests directly. */
svdq_status svdq_debug_group_sums(const svdq_layer* layer, int64_t M, int32_t form, const uint8_t* qX,
                                  int64_t m0, int64_t n0, int64_t mt, int64_t nt, int32_t* out,
                                  void* stream);

#ifdef __cplusplus
}
#endif
#endif /* SVDQ_H */
