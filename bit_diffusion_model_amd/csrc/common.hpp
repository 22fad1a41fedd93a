// Shared device helpers for the gfx950 kernels of the SVDQuant W4A4 layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace svdq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));

constexpr int kMaxRank = 128;

__device__ __forceinline__ float bf16_lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Round-to-nearest-even fp32 -> bf16 bits (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Expand 8 sign-magnitude 4-bit codes (one dword, element 2j in the low nibble of
// byte j) into 8 FP8 E4M3 bytes whose value is q * 2^-9: with a zero exponent field
// the E4M3 mantissa bits hold |q| directly (subnormal), and bit 7 is the sign.
// lo receives elements 0,2,4,6 (low nibbles), hi receives elements 1,3,5,7.
__device__ __forceinline__ void nib8_to_fp8(uint32_t d, uint32_t& lo, uint32_t& hi) {
  lo = (d & 0x07070707u) | ((d & 0x08080808u) << 4);
  hi = ((d >> 4) & 0x07070707u) | (d & 0x80808080u);
}

// The same expansion for the kernel's weight layout, in which each byte j of the word
// holds element 2j in bits 0-2 (magnitude) and 7 (sign), the magnitude of element 2j+1
// in bits 4-6, and in bit 3 the sign of element 2j-1 (cyclically, of byte j-1's odd
// element).  Then lo is a mask, and hi is the word rotated by 4 bits and masked.
__device__ __forceinline__ void nib8p_to_fp8(uint32_t d, uint32_t& lo, uint32_t& hi) {
  lo = d & 0x87878787u;
  hi = __builtin_amdgcn_alignbit(d, d, 4) & 0x87878787u;
}

// An INT4 group scale s = m * 2^e (m in [1, 2)), given as fp32 bits (every fp16 value
// is exact in fp32), as one word: bits 0-15 the fp16 m (0 for s = 0), bits 16-23 the
// E8M0 byte of 2^(e + 9) (127 for s = 0).  2^-9 is the value of FP8 code 1, so an MFMA
// with these block scales on both sides returns the exact integer group sum times
// 2^(eX + eW).
__device__ __forceinline__ uint32_t split_scale_f32(uint32_t u) {
  const float f = __uint_as_float(u);
  const uint32_t m = f == 0.0f ? 0u : __builtin_bit_cast(uint16_t, (_Float16)__uint_as_float((u & 0x807FFFFFu) | (127u << 23)));
  const uint32_t eb = f == 0.0f ? 127u : ((u >> 23) & 0xFFu) + 9u;
  return m | (eb << 16);
}
// The same from fp16 bits.
__device__ __forceinline__ uint32_t split_scale_word(uint32_t bits) {
  return split_scale_f32(__float_as_uint((float)__builtin_bit_cast(_Float16, (uint16_t)bits)));
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
__device__ __forceinline__ void buf_store2(uint16_t v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b16(v, r, off, 0, 0);
}

__device__ __forceinline__ float wave_max_xor(float v, int mask) {
  return fmaxf(v, __shfl_xor(v, mask, 64));
}

}  // namespace svdq
