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

// The value of lane l and of lane l ^ 16 (resp. l ^ 32), through the gfx950
// row-swap instructions (VALU, no LDS): with both operands equal,
// v_permlane16_swap returns the even row of each pair of rows in its first
// result and the odd row in its second, in every lane; v_permlane32_swap
// does the same for the two halves of the wave.
__device__ __forceinline__ void pair_xor16(float v, float &a, float &b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v),
                                                  false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void pair_xor32(float v, float &a, float &b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                  false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
// max / sum over the 4 lanes l, l^16, l^32, l^48; every lane gets the same
// value (the two operands of each step are the same pair in every lane).
__device__ __forceinline__ float max_over_rows(float v) {
  float a, b;
  pair_xor16(v, a, b);
  v = fmaxf(a, b);
  pair_xor32(v, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float sum_over_rows(float v) {
  float a, b;
  pair_xor16(v, a, b);
  v = a + b;
  pair_xor32(v, a, b);
  return a + b;
}

// Cross-lane steps on the DPP network (register-to-register, no LDS round
// trip).  dpp_row<ctrl>(old, src): the src value of the lane `ctrl` selects
// inside the same row of 16 lanes; lanes whose source falls outside the row
// keep `old`.
template <int kCtrl>
__device__ __forceinline__ uint32_t dpp_row(uint32_t old, uint32_t src) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)src, kCtrl, 0xf, 0xf, false);
}
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;

__device__ __forceinline__ uint32_t lane_id() { return threadIdx.x & (kWave - 1); }

// Inclusive prefix sum over the 64 lanes of a wave (all lanes active).
__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t x) {
  x += dpp_row<kRowShr1>(0u, x);       // scan inside each row of 16
  x += dpp_row<kRowShr2>(0u, x);
  x += dpp_row<kRowShr4>(0u, x);
  x += dpp_row<kRowShr8>(0u, x);
  const uint32_t r0 = __builtin_amdgcn_readlane(x, 15);   // row totals
  const uint32_t r1 = __builtin_amdgcn_readlane(x, 31);
  const uint32_t r2 = __builtin_amdgcn_readlane(x, 47);
  const uint32_t row = lane_id() >> 4;
  return x + (row >= 1 ? r0 : 0u) + (row >= 2 ? r1 : 0u) + (row >= 3 ? r2 : 0u);
}

// Wave-wide min / max of uint32 (all lanes active); the result is uniform.
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
  x = min(x, dpp_row<kRowShr1>(x, x));
  x = min(x, dpp_row<kRowShr2>(x, x));
  x = min(x, dpp_row<kRowShr4>(x, x));
  x = min(x, dpp_row<kRowShr8>(x, x));
  return min(min((uint32_t)__builtin_amdgcn_readlane(x, 15), (uint32_t)__builtin_amdgcn_readlane(x, 31)),
             min((uint32_t)__builtin_amdgcn_readlane(x, 47), (uint32_t)__builtin_amdgcn_readlane(x, 63)));
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = max(x, dpp_row<kRowShr1>(x, x));
  x = max(x, dpp_row<kRowShr2>(x, x));
  x = max(x, dpp_row<kRowShr4>(x, x));
  x = max(x, dpp_row<kRowShr8>(x, x));
  return max(max((uint32_t)__builtin_amdgcn_readlane(x, 15), (uint32_t)__builtin_amdgcn_readlane(x, 31)),
             max((uint32_t)__builtin_amdgcn_readlane(x, 47), (uint32_t)__builtin_amdgcn_readlane(x, 63)));
}

// Pages of a request of ctx tokens, limited to the page-table row.
__device__ __forceinline__ int pages_in(int ctx, int page_size, int max_pages) {
  int n = ctx <= 0 ? 0 : (ctx + page_size - 1) / page_size;
  return n < max_pages ? n : max_pages;
}

}  // namespace quest
