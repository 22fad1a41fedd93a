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

__device__ __forceinline__ float wave_max_xor(float v, int mask) {
  return fmaxf(v, __shfl_xor(v, mask, 64));
}

}  // namespace svdq
