// Hardware-cost microbenchmarks behind the kernel design notes (gfx950, timing only;
// every access in bounds).  Prints one JSON object per line:
//   {"what": ..., "waves_per_simd": ..., "cycles": ...}    cycles per unit at 2.4 GHz
//   {"what": ..., "bytes_per_cycle_cu": ...}              per CU at 2.4 GHz
//   {"what": "mfma_32x32x4_2b_f16_layout", "ok": 0|1}    operand / result layout probe
//   {"what": "cross_...", "nv": ..., "cycles_per_iter": ...}  per SIMD at 2.4 GHz
//   {"what": "valu_<instruction>", "waves_per_simd": ..., "cycles": ...}  per instruction
// Units: one MFMA (MFMA chains), one VALU instruction (VALU only), one MFMA plus its
// VALU (same-wave overlap), one tile and group (the INT4 rescale pattern: group-sum
// MFMA, scale-product MFMA, 16 v_fmac); cross_*: one iteration of two FP6 MFMAs in one
// wave and / or nv v_fmac in another wave of the same SIMD.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <vector>

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v32f __attribute__((ext_vector_type(32)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));

#define CHECK(x)                                                                     \
  do {                                                                               \
    hipError_t e_ = (x);                                                             \
    if (e_ != hipSuccess) {                                                          \
      fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      exit(1);                                                                       \
    }                                                                                \
  } while (0)

constexpr int ITER = 2048;

// MODE 0: FP6 32x32x64 scaled MFMA, 4 independent chains
// MODE 1: FP8 32x32x64 scaled MFMA, 4 chains
// MODE 2: f16 32x32x8 MFMA, 4 chains
// MODE 3: VALU only, NV v_fmac per iteration
// MODE 4: same wave: FP6 MFMA + NV independent v_fmac, twice per iteration
// MODE 5: the INT4 rescale pattern for two tiles: scale MFMA, group-sum MFMA, 16 v_fmac each
template <int MODE, int NV>
__global__ void kcost(float* out, int seed) {
  const int lane = threadIdx.x & 63;
  v8i a = {lane + seed, 3, 5, 7, 9, 11, 0, 0};
  v8i b = {lane * 3 + seed, 1, 2, 3, 4, 5, 0, 0};
  v16f acc0 = {}, acc1 = {}, acc2 = {}, acc3 = {};
  float x[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) x[i] = (float)(lane + i) * 1e-3f;
  const float y = 1.0001f + seed * 1e-7f;
  v4h ha = {(_Float16)1.0f, 0, 0, 0}, hb = {(_Float16)(0.5f + lane * 1e-3f), 0, 0, 0};
  for (int it = 0; it < ITER; ++it) {
    if constexpr (MODE == 0 || MODE == 1) {
      constexpr int F = MODE == 0 ? 2 : 0;
      acc0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc0, F, F, 0, 127, 0, 127);
      acc1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc1, F, F, 0, 127, 0, 127);
      acc2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc2, F, F, 0, 127, 0, 127);
      acc3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc3, F, F, 0, 127, 0, 127);
    } else if constexpr (MODE == 2) {
      acc0 = __builtin_amdgcn_mfma_f32_32x32x8f16(ha, hb, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x8f16(hb, ha, acc1, 0, 0, 0);
      acc2 = __builtin_amdgcn_mfma_f32_32x32x8f16(ha, ha, acc2, 0, 0, 0);
      acc3 = __builtin_amdgcn_mfma_f32_32x32x8f16(hb, hb, acc3, 0, 0, 0);
    } else if constexpr (MODE == 3) {
#pragma unroll
      for (int i = 0; i < NV; ++i) x[i % 32] = fmaf(x[i % 32], y, 1e-9f);
    } else if constexpr (MODE == 4) {
      acc0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc0, 2, 2, 0, 127, 0, 127);
#pragma unroll
      for (int i = 0; i < NV; ++i) x[i % 32] = fmaf(x[i % 32], y, 1e-9f);
      acc1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc1, 2, 2, 0, 127, 0, 127);
#pragma unroll
      for (int i = 0; i < NV; ++i) x[(i + 16) % 32] = fmaf(x[(i + 16) % 32], y, 1e-9f);
    } else {
      const v16f c0 = __builtin_amdgcn_mfma_f32_32x32x8f16(ha, hb, v16f{}, 0, 0, 0);
      const v16f p0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, v16f{}, 2, 2, 0, 130, 0, 130);
      const v16f c1 = __builtin_amdgcn_mfma_f32_32x32x8f16(hb, ha, v16f{}, 0, 0, 0);
      const v16f p1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, v16f{}, 2, 2, 0, 130, 0, 130);
#pragma unroll
      for (int i = 0; i < 16; ++i) acc0[i] = fmaf(p0[i], c0[i], acc0[i]);
#pragma unroll
      for (int i = 0; i < 16; ++i) acc1[i] = fmaf(p1[i], c1[i], acc1[i]);
      a[0] += 1;
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += acc0[i] + acc1[i] + acc2[i] + acc3[i];
#pragma unroll
  for (int i = 0; i < 32; ++i) s += x[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

static float best_ms(void (*launch)(void*), void* arg) {
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  launch(arg);
  CHECK(hipDeviceSynchronize());
  float best = 1e30f;
  for (int r = 0; r < 5; ++r) {
    CHECK(hipEventRecord(e0));
    launch(arg);
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    float ms;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    if (ms < best) best = ms;
  }
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
  return best;
}

// VALU issue cost of one instruction class: 32 independent registers per lane, one
// instruction of the class on each per iteration (inline asm, so the instruction is the
// one named).  OP: 0 v_fmac_f32, 1 v_mul_f32, 2 v_and_b32, 3 v_add_f32, 4 v_fma_mix_f32,
// 5 v_pk_mul_f16, 6 v_lshlrev_b32, 7 v_alignbit_b32, 8 v_cvt_f32_f16.
template <int OP>
__global__ void kvalu(float* out, int seed) {
  const int lane = threadIdx.x & 63;
  uint32_t x[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) x[i] = __float_as_uint((float)(lane + i + seed) * 1e-3f);
  const uint32_t y = __float_as_uint(1.0001f), z = __float_as_uint(1e-9f);
  for (int it = 0; it < ITER; ++it) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if constexpr (OP == 0) asm volatile("v_fmac_f32 %0, %1, %2" : "+v"(x[i]) : "v"(y), "v"(z));
      else if constexpr (OP == 1) asm volatile("v_mul_f32 %0, %0, %1" : "+v"(x[i]) : "v"(y));
      else if constexpr (OP == 2) asm volatile("v_and_b32 %0, %0, %1" : "+v"(x[i]) : "v"(y));
      else if constexpr (OP == 3) asm volatile("v_add_f32 %0, %0, %1" : "+v"(x[i]) : "v"(z));
      else if constexpr (OP == 4) asm volatile("v_fma_mix_f32 %0, %0, %1, %2" : "+v"(x[i]) : "v"(y), "v"(z));
      else if constexpr (OP == 5) asm volatile("v_pk_mul_f16 %0, %0, %1" : "+v"(x[i]) : "v"(y));
      else if constexpr (OP == 6) asm volatile("v_lshlrev_b32 %0, 1, %0" : "+v"(x[i]));
      else if constexpr (OP == 7) asm volatile("v_alignbit_b32 %0, %0, %1, 8" : "+v"(x[i]) : "v"(y));
      else asm volatile("v_cvt_f32_f16 %0, %0" : "+v"(x[i]));
    }
  }
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) s ^= x[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = (float)s;
}

struct CostArg {
  float* out;
  int blocks;
};
template <int MODE, int NV>
static void launch_cost(void* p) {
  const CostArg* c = static_cast<const CostArg*>(p);
  hipLaunchKernelGGL((kcost<MODE, NV>), dim3(c->blocks), dim3(256), 0, 0, c->out, 1);
}

template <int OP>
static void launch_valu(void* p) {
  const CostArg* c = static_cast<const CostArg*>(p);
  hipLaunchKernelGGL((kvalu<OP>), dim3(c->blocks), dim3(256), 0, 0, c->out, 1);
}
template <int OP>
static void valu_cost(const char* what, int blocks_per_cu) {
  CostArg a{nullptr, 256 * blocks_per_cu};
  CHECK(hipMalloc(&a.out, (size_t)a.blocks * 256 * sizeof(float)));
  const float ms = best_ms(launch_valu<OP>, &a);
  CHECK(hipFree(a.out));
  const double cycles = ms * 1e-3 * 2.4e9 / ((double)ITER * blocks_per_cu * 32);
  printf("{\"what\": \"valu_%s\", \"waves_per_simd\": %d, \"cycles\": %.1f}\n", what, blocks_per_cu, cycles);
}
template <int OP>
static void valu_both(const char* what) {
  valu_cost<OP>(what, 2);
  valu_cost<OP>(what, 8);
}

// waves_per_simd = blocks per CU (4 waves per block, one per SIMD)
template <int MODE, int NV>
static void cost(const char* what, int blocks_per_cu, double units_per_iter) {
  CostArg a{nullptr, 256 * blocks_per_cu};
  CHECK(hipMalloc(&a.out, (size_t)a.blocks * 256 * sizeof(float)));
  const float ms = best_ms(launch_cost<MODE, NV>, &a);
  CHECK(hipFree(a.out));
  const double cycles = ms * 1e-3 * 2.4e9 / (ITER * blocks_per_cu * units_per_iter);
  printf("{\"what\": \"%s\", \"waves_per_simd\": %d, \"cycles\": %.1f}\n", what, blocks_per_cu, cycles);
}

// 32x32x4 f16 with two blocks: block b takes A rows / B columns from lanes 32 b .. 32 b + 31
// and writes result registers 16 b .. 16 b + 15 in the single-block layout (lane l holds
// column l & 31, rows 8 (r >> 2) + 4 (l >> 5) + (r & 3) of its block).
__global__ void probe2b(float* out, int which) {
  const int l = threadIdx.x;
  v4h a = {0, 0, 0, 0}, b = {0, 0, 0, 0};
  if (which == 0) {
    a[0] = (_Float16)(l + 1);
    b[0] = (_Float16)1.0f;
  } else {
    a[0] = (_Float16)1.0f;
    b[0] = (_Float16)(l + 1);
  }
  const v32f d = __builtin_amdgcn_mfma_f32_32x32x4f16(a, b, v32f{}, 0, 0, 0);
  for (int i = 0; i < 32; ++i) out[l * 32 + i] = d[i];
}

static void layout_2b() {
  float* d;
  CHECK(hipMalloc(&d, 64 * 32 * sizeof(float)));
  std::vector<float> h(64 * 32);
  bool ok = true;
  for (int which = 0; which < 2; ++which) {
    hipLaunchKernelGGL(probe2b, dim3(1), dim3(64), 0, 0, d, which);
    CHECK(hipMemcpy(h.data(), d, h.size() * sizeof(float), hipMemcpyDeviceToHost));
    for (int l = 0; l < 64; ++l)
      for (int r = 0; r < 32; ++r) {
        const int blk = r >> 4, a = r & 15;
        const int row = 8 * (a >> 2) + 4 * (l >> 5) + (a & 3), col = l & 31;
        const float want = which == 0 ? (float)(32 * blk + row + 1) : (float)(32 * blk + col + 1);
        if (h[l * 32 + r] != want) ok = false;
      }
  }
  CHECK(hipFree(d));
  printf("{\"what\": \"mfma_32x32x4_2b_f16_layout\", \"ok\": %d}\n", ok ? 1 : 0);
}

// LDS-destination buffer loads (16 bytes per lane), NB in flight per wave; a wave's
// window is 32 KB of a 2 MB region (L2-resident) or its own slice of 1 GiB (from HBM).
template <int NB, bool L2>
__global__ __launch_bounds__(256) void kdma(const uint8_t* __restrict__ src, size_t per_wave, int reps, float* out) {
  __shared__ __attribute__((aligned(1024))) uint8_t ring[4][NB][1024];
  // wave-uniform (readfirstlane): a per-lane wave index makes the buffer resource look
  // divergent, and the compiler then wraps every load in a waterfall loop
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const size_t gw = (size_t)blockIdx.x * 4 + wave;
  const uint8_t* base = L2 ? src + (gw % 64) * 32768 : src + gw * per_wave;
  const int bytes = L2 ? 32768 : (int)per_wave;
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0, bytes, 0x00020000);
  const int n = L2 ? reps : (int)(per_wave / 1024);
  for (int i = 0; i < n; ++i) {
    const uint32_t off = (uint32_t)((L2 ? (i % 32) : i) * 1024 + lane * 16);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)&ring[wave][i % NB][0], 16,
                                             off, 0, 0, 0);
    if (i >= NB - 1) __builtin_amdgcn_s_waitcnt((NB - 1) | (7 << 4) | (15 << 8));
  }
  __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));
  __syncthreads();
  out[gw * 64 + lane] = (float)ring[wave][lane % NB][lane];
}

// The same stream through registers: 16-byte buffer loads (8 in flight per wave), each
// written to LDS with ds_write_b128 once it has arrived (the asm store keeps the compiler
// from dropping the otherwise unread LDS data).
typedef unsigned v4u __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) void kreg(const uint8_t* __restrict__ src, int reps, float* out) {
  __shared__ __attribute__((aligned(1024))) uint8_t ring[4][8][1024];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const size_t gw = (size_t)blockIdx.x * 4 + wave;
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(src + (gw % 64) * 32768), (short)0, 32768, 0x00020000);
  v4u reg[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) reg[j] = __builtin_amdgcn_raw_buffer_load_b128(r, (uint32_t)(j * 1024 + lane * 16), 0, 0);
  for (int i = 8; i < reps; i += 8) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      asm volatile("ds_write_b128 %0, %1" ::"v"((uint32_t)(uintptr_t)&ring[wave][j][lane * 16]), "v"(reg[j]) : "memory");
      reg[j] = __builtin_amdgcn_raw_buffer_load_b128(r, (uint32_t)(((i + j) % 32) * 1024 + lane * 16), 0, 0);
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j)
    asm volatile("ds_write_b128 %0, %1" ::"v"((uint32_t)(uintptr_t)&ring[wave][j][lane * 16]), "v"(reg[j]) : "memory");
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  out[gw * 64 + lane] = (float)ring[wave][lane % 8][lane];
}

struct DmaArg {
  const uint8_t* src;
  size_t per_wave;
  int reps, blocks;
  float* out;
};
template <int NB, bool L2>
static void launch_dma(void* p) {
  const DmaArg* a = static_cast<const DmaArg*>(p);
  hipLaunchKernelGGL((kdma<NB, L2>), dim3(a->blocks), dim3(256), 0, 0, a->src, a->per_wave, a->reps, a->out);
}

template <int NB, bool L2>
static void dma(const uint8_t* src, size_t total, int blocks_per_cu) {
  DmaArg a{src, 0, 4096, 256 * blocks_per_cu, nullptr};
  a.per_wave = total / ((size_t)a.blocks * 4) / 1024 * 1024;
  CHECK(hipMalloc(&a.out, (size_t)a.blocks * 4 * 64 * sizeof(float)));
  const float ms = best_ms(launch_dma<NB, L2>, &a);
  CHECK(hipFree(a.out));
  const double bytes = L2 ? (double)a.reps * 1024 * a.blocks * 4 : (double)a.per_wave * a.blocks * 4;
  printf("{\"what\": \"lds_dma_%s_%d_in_flight_%d_blocks\", \"bytes_per_cycle_cu\": %.1f}\n", L2 ? "l2" : "hbm", NB,
         blocks_per_cu, bytes / (ms * 1e-3) / 256 / 2.4e9);
}

static void launch_reg(void* p) {
  const DmaArg* a = static_cast<const DmaArg*>(p);
  hipLaunchKernelGGL(kreg, dim3(a->blocks), dim3(256), 0, 0, a->src, a->reps, a->out);
}

static void regload(const uint8_t* src, int blocks_per_cu) {
  DmaArg a{src, 0, 4096, 256 * blocks_per_cu, nullptr};
  CHECK(hipMalloc(&a.out, (size_t)a.blocks * 4 * 64 * sizeof(float)));
  const float ms = best_ms(launch_reg, &a);
  CHECK(hipFree(a.out));
  const double bytes = (double)a.reps * 1024 * a.blocks * 4;
  printf("{\"what\": \"reg_load_ds_write_l2_8_in_flight_%d_blocks\", \"bytes_per_cycle_cu\": %.1f}\n", blocks_per_cu,
         bytes / (ms * 1e-3) / 256 / 2.4e9);
}

// MFMA and VALU in different waves of one SIMD: a block of 8 waves, wave w on SIMD w % 4;
// waves 0-3 run FP6 MFMA chains (two per iteration), waves 4-7 NV v_fmac per iteration.
// role 0: the wave exits at once.
template <int NV>
__global__ __launch_bounds__(512) void kcross(float* out, int roleA, int roleB) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int role = wave < 4 ? roleA : roleB;
  float s = 0.f;
  if (role == 1) {
    v8i a = {lane, 3, 5, 7, 9, 11, 0, 0}, b = {lane * 3, 1, 2, 3, 4, 5, 0, 0};
    v16f acc0 = {}, acc1 = {};
    for (int it = 0; it < ITER; ++it) {
      acc0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc0, 2, 2, 0, 130, 0, 130);
      acc1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc1, 2, 2, 0, 130, 0, 130);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc0[i] + acc1[i];
  } else if (role == 2) {
    float x[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] = (float)(lane + i) * 1e-3f;
    for (int it = 0; it < ITER; ++it) {
#pragma unroll
      for (int i = 0; i < NV; ++i) x[i % 32] = fmaf(x[i % 32], 1.0001f, 1e-9f);
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) s += x[i];
  }
  out[blockIdx.x * 512 + threadIdx.x] = s;
}

struct CrossArg {
  float* out;
  int ra, rb;
};
template <int NV>
static void launch_cross(void* p) {
  const CrossArg* c = static_cast<const CrossArg*>(p);
  hipLaunchKernelGGL((kcross<NV>), dim3(256), dim3(512), 0, 0, c->out, c->ra, c->rb);
}
template <int NV>
static void cross(const char* what, int ra, int rb) {
  CrossArg a{nullptr, ra, rb};
  CHECK(hipMalloc(&a.out, (size_t)256 * 512 * sizeof(float)));
  const float ms = best_ms(launch_cross<NV>, &a);
  CHECK(hipFree(a.out));
  printf("{\"what\": \"%s\", \"nv\": %d, \"cycles_per_iter\": %.1f}\n", what, NV, ms * 1e-3 * 2.4e9 / ITER);
}

// ds_read_b128 bandwidth: consecutive lanes read consecutive 16-byte slots
__global__ __launch_bounds__(1024) void klds(float* out, int reps) {
  __shared__ __attribute__((aligned(16))) uint4 buf[4096];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < 4096; i += blockDim.x) buf[i] = make_uint4(i, i + 1, i + 2, i + 3);
  __syncthreads();
  uint4 acc = make_uint4(0, 0, 0, 0);
  for (int r = 0; r < reps; ++r) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint4 v = buf[((wave * 8 + k + r) & 63) * 64 + lane];
      acc.x ^= v.x;
      acc.y ^= v.y;
      acc.z ^= v.z;
      acc.w ^= v.w;
    }
  }
  out[blockIdx.x * blockDim.x + tid] = (float)(acc.x + acc.y + acc.z + acc.w);
}

struct LdsArg {
  int waves;
  float* out;
};
static void launch_lds(void* p) {
  const LdsArg* a = static_cast<const LdsArg*>(p);
  hipLaunchKernelGGL(klds, dim3(256), dim3(64 * a->waves), 0, 0, a->out, 4096);
}

static void lds(int waves) {
  LdsArg a{waves, nullptr};
  CHECK(hipMalloc(&a.out, (size_t)256 * 64 * waves * sizeof(float)));
  const float ms = best_ms(launch_lds, &a);
  CHECK(hipFree(a.out));
  const double bytes = 4096.0 * 8 * 1024 * waves * 256;
  printf("{\"what\": \"ds_read_b128_%d_waves_per_cu\", \"bytes_per_cycle_cu\": %.1f}\n", waves,
         bytes / (ms * 1e-3) / 256 / 2.4e9);
}

int main() {
  cost<0, 0>("mfma_fp6_32x32x64", 1, 4);
  cost<0, 0>("mfma_fp6_32x32x64", 2, 4);
  cost<1, 0>("mfma_fp8_32x32x64", 1, 4);
  cost<2, 0>("mfma_f16_32x32x8", 2, 4);
  cost<3, 32>("valu_fmac", 1, 32);
  cost<3, 32>("valu_fmac", 2, 32);
  cost<4, 0>("same_wave_fp6_mfma_plus_0_fmac", 1, 2);
  cost<4, 8>("same_wave_fp6_mfma_plus_8_fmac", 1, 2);
  cost<4, 16>("same_wave_fp6_mfma_plus_16_fmac", 1, 2);
  cost<4, 16>("same_wave_fp6_mfma_plus_16_fmac", 2, 2);
  cost<5, 0>("int4_rescale_tile_group", 1, 2);
  cost<5, 0>("int4_rescale_tile_group", 2, 2);
  layout_2b();
  const size_t total = (size_t)1 << 30;
  uint8_t* src;
  CHECK(hipMalloc(&src, total));
  CHECK(hipMemset(src, 1, total));
  CHECK(hipDeviceSynchronize());
  dma<8, false>(src, total, 1);
  dma<8, true>(src, total, 1);
  dma<8, true>(src, total, 2);
  regload(src, 1);
  regload(src, 2);
  CHECK(hipFree(src));
  cross<16>("cross_mfma_only", 1, 0);
  cross<16>("cross_valu_only", 0, 2);
  cross<16>("cross_mfma_and_valu_waves", 1, 2);
  valu_both<0>("v_fmac_f32");
  valu_both<1>("v_mul_f32");
  valu_both<2>("v_and_b32");
  valu_both<3>("v_add_f32");
  valu_both<4>("v_fma_mix_f32");
  valu_both<5>("v_pk_mul_f16");
  valu_both<6>("v_lshlrev_b32");
  valu_both<7>("v_alignbit_b32");
  valu_both<8>("v_cvt_f32_f16");
  lds(4);
  lds(8);
  lds(16);
  return 0;
}
