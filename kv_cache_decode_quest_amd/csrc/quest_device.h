// quest_device.h -- device helpers shared by the gfx950 kernels of libquest.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace quest {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// bf16 <-> fp32.  bf16 is the upper half of a binary32, so widening is exact.
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16 with round to nearest, ties to even (NaN stays a quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Element access for the two storage types.
template <typename T> struct Elem;
template <> struct Elem<float> {
  using storage = float;
  __device__ __forceinline__ static float load(const float *p, int64_t i) { return p[i]; }
  __device__ __forceinline__ static void store(float *p, int64_t i, float x) { p[i] = x; }
};
template <> struct Elem<uint16_t> {
  using storage = uint16_t;
  __device__ __forceinline__ static float load(const uint16_t *p, int64_t i) {
    return bf16_bits_to_f32(p[i]);
  }
  __device__ __forceinline__ static void store(uint16_t *p, int64_t i, float x) {
    p[i] = (uint16_t)f32_to_bf16_bits(x);
  }
};

// Wave-wide reductions over lanes whose index differs in the given bits.
__device__ __forceinline__ float wave_max_xor(float v, int mask) {
  return fmaxf(v, __shfl_xor(v, mask, kWave));
}

// Pages of a request of ctx tokens, limited to the page-table row.
__device__ __forceinline__ int pages_in(int ctx, int page_size, int max_pages) {
  int n = ctx <= 0 ? 0 : (ctx + page_size - 1) / page_size;
  return n < max_pages ? n : max_pages;
}

}  // namespace quest
