// Shared device helpers for the gfx950 kernels of the SVDQuant W4A4 layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace svdq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v6i __attribute__((ext_vector_type(6)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v2i_t __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));

constexpr int kMaxRank = 128;

__device__ __forceinline__ float bf16_lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Round-to-nearest-even fp32 -> bf16 bits (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// An empty asm statement that reads v: v stays live (in its registers) up to this point.
// Used after v_cvt_scalef32_2xpk16_fp6_f32, whose six result registers must not overlap
// its 32 source registers: measured on gfx950, a result register allocated on top of a
// source register at a higher position than its own is written before that source is
// read (the instruction converts in passes), corrupting the codes that source carries.
// The compiler does not mark the result early-clobber, so keeping the sources live past
// the instruction is what keeps the allocator from overlapping them.
template <typename T>
__device__ __forceinline__ void keep_live(const T& v) {
  asm volatile("" ::"v"(v));
}

// Expand 8 sign-magnitude 4-bit codes (one dword, element 2j in the low nibble of
// byte j) into 8 FP8 E4M3 bytes whose value is q * 2^-9: with a zero exponent field
// the E4M3 mantissa bits hold |q| directly (subnormal), and bit 7 is the sign.
// lo receives elements 0,2,4,6 (low nibbles), hi receives elements 1,3,5,7.
__device__ __forceinline__ void nib8_to_fp8(uint32_t d, uint32_t& lo, uint32_t& hi) {
  lo = (d & 0x07070707u) | ((d & 0x08080808u) << 4);
  hi = ((d >> 4) & 0x07070707u) | (d & 0x80808080u);
}

// INT4 codes as matrix-core FP6 E2M3 operands: code q is the 6-bit field sign << 5 | |q|
// (exponent 0: the value q / 8).  One operand half (32 codes of a group half) is six
// words with field f at bit 6 f; field f carries k = 16 (f & 1) + (f >> 1) of the half.
// Bits 3-4 of every field are zero, so the prepared weight layout stores the half in
// four words w0..w3 with the info bits of words 2 and 5 on the zero bits of words
// 0, 1 and 3, 4: w0 = f0 | (f2 & Z0), w1 = f1 | (f2 & Z1) (and w2, w3 from f3, f4, f5).
constexpr uint32_t kZ0 = (3u << 3) | (3u << 9) | (3u << 15) | (3u << 21) | (3u << 27);
constexpr uint32_t kZ1 = (3u << 1) | (3u << 7) | (3u << 13) | (3u << 19) | (3u << 25) | (1u << 31);
__device__ __forceinline__ v8i expand_w6(uint4 w) {
  return v8i{(int)(w.x & ~kZ0), (int)(w.y & ~kZ1), (int)((w.x & kZ0) | (w.y & kZ1)),
             (int)(w.z & ~kZ0), (int)(w.w & ~kZ1), (int)((w.z & kZ0) | (w.w & kZ1)), 0, 0};
}

// 32 sign-magnitude nibbles of a group half in storage order (code 2j in the low nibble
// of byte j) -> the six FP6 operand words: nibbles -> FP8 bytes q * 2^-9 -> fp32 ->
// the FP6 converter (x / 2^-6 = q / 8, exact), which interleaves its two 16-value inputs
// field by field (codes 0-15 in the even fields, 16-31 in the odd ones).
__device__ __forceinline__ v6i nib32_to_fp6(uint4 d) {
  const uint32_t dw[4] = {d.x, d.y, d.z, d.w};
  v16f x0, x1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t lo, hi;
    nib8_to_fp8(dw[i], lo, hi);  // lo: codes 8i + 0, 2, 4, 6; hi: 8i + 1, 3, 5, 7
    const v2f a = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, false), b = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, true);
    const v2f c = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, false), e = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, true);
    const float v[8] = {a.x, c.x, a.y, c.y, b.x, e.x, b.y, e.y};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (i < 2) x0[8 * i + j] = v[j];
      else x1[8 * (i - 2) + j] = v[j];
    }
  }
  const v6i r = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(x0, x1, 0x1p-6f);
  keep_live(x0);
  keep_live(x1);
  return r;
}

// Eight E2M1 codes (one dword, code 2j in the low nibble of byte j) times a group scale
// s > 0 -> eight fp16 values, in code order, exact (at most 6 significant bits, binary
// exponents -10 .. 11).  The scaled FP4 conversion applies only the exponent of its fp32
// scale (2^floor(log2 s), measured), so the mantissa ratio s / 2^floor(log2 s) (1 to 1.875)
// is applied after it with a packed fp16 multiply.  s = 0 gives zeros.
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
__device__ __forceinline__ v8h nv_f16x8(uint32_t w, float s) {
  const float r = __uint_as_float((__float_as_uint(s) & 0x007FFFFFu) | 0x3F800000u);
  const h2 rr = {(_Float16)r, (_Float16)r};
  const h2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s, 0) * rr;
  const h2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s, 1) * rr;
  const h2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s, 2) * rr;
  const h2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s, 3) * rr;
  return v8h{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

// GELU in its exact form, x Phi(x) with Phi(x) = erfc(-x / sqrt 2) / 2, in fp32.  erfc(z)
// for z >= 0 by the Chebyshev fit of Numerical Recipes (Press et al., "Incomplete gamma
// function, error function", routine erfcc; fractional error below 1.2e-7 for z >= 0):
// erfc(z) = t exp(-z^2 + P(t)), t = 1 / (1 + z / 2), P a degree-9 polynomial whose
// constant term here also carries -ln 2, so the exponential gives erfc / 2 directly; for
// x >= 0, Phi(x) = 1 - erfc(x / sqrt 2) / 2.  Evaluated in fp32 the relative error of
// GELU stays below 2e-5 (the exponential's argument reaches -z^2), far inside the bf16
// rounding that follows; the tail keeps its relative accuracy (no 1 + erf cancellation).
__device__ __forceinline__ float gelu_erf(float x) {
  const float z = fabsf(x) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(0.5f, z, 1.0f));
  float p = 0.17087277f;
  p = fmaf(p, t, -0.82215223f);
  p = fmaf(p, t, 1.48851587f);
  p = fmaf(p, t, -1.13520398f);
  p = fmaf(p, t, 0.27886807f);
  p = fmaf(p, t, -0.18628806f);
  p = fmaf(p, t, 0.09678418f);
  p = fmaf(p, t, 0.37409196f);
  p = fmaf(p, t, 1.00002368f);
  p = fmaf(p, t, -1.95865941f);  // -1.26551223 - ln 2
  const float h = t * __expf(fmaf(-z, z, p));  // erfc(|x| / sqrt 2) / 2
  return x * (x >= 0.0f ? 1.0f - h : h);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
// bf16(GELU(a)) in the low half, bf16(GELU(b)) in the high half (hardware conversion,
// round to nearest even)
__device__ __forceinline__ uint32_t gelu_bf16x2(float a, float b) {
  const bf16x2_t v = {(__bf16)gelu_erf(a), (__bf16)gelu_erf(b)};
  return __builtin_bit_cast(uint32_t, v);
}

// Raw buffer resource over `bytes` bytes at p: loads beyond the range return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ uint32_t buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t buf_load2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t buf_load1(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
}
// Stores through a buffer resource: a store whose offset is outside the range is
// dropped (the offset is checked in full; nothing goes through the scalar offset).
__device__ __forceinline__ void buf_store4(uint32_t v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, 0);
}
__device__ __forceinline__ void buf_store16(uint4 v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i, v), r, off, 0, 0);
}
__device__ __forceinline__ void buf_store8(uint2 v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(v2i_t, v), r, off, 0, 0);
}
__device__ __forceinline__ void buf_store1(uint8_t v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b8(v, r, off, 0, 0);
}
// An offset no buffer of this library reaches: a store given it is dropped by the range
// check, so a lane that must not store still issues the (unconditional) instruction.
constexpr uint32_t kNoStore = 0xFFFFFFF0u;
__device__ __forceinline__ void buf_store2(uint16_t v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b16(v, r, off, 0, 0);
}

__device__ __forceinline__ float wave_max_xor(float v, int mask) {
  return fmaxf(v, __shfl_xor(v, mask, 64));
}

}  // namespace svdq
