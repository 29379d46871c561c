// Shared device helpers for the LoopVQ HIP kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace loopvq {

constexpr int kWave = 64;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round-to-nearest-even float -> bf16 bits (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// fp16 bits -> double, exact.
__device__ __forceinline__ double f16_bits_to_f64(uint16_t h) {
  _Float16 v;
  __builtin_memcpy(&v, &h, 2);
  return (double)(float)v;
}

// fp64 -> fp16 bits, round to nearest even (finite inputs; overflow saturates
// to the largest finite value).
__device__ __forceinline__ uint16_t f64_to_f16_rne(double v) {
  const uint16_t sign = v < 0.0 ? 0x8000 : 0;
  const double av = fabs(v);
  const _Float16 h0 = (_Float16)(float)av;
  uint16_t b0;
  __builtin_memcpy(&b0, &h0, 2);
  if (b0 >= 0x7c00) b0 = 0x7bff;
  uint16_t best = b0;
  double bestd = fabs(av - f16_bits_to_f64(b0));
  for (int k = -1; k <= 1; k += 2) {
    const int c = (int)b0 + k;
    if (c < 0 || c >= 0x7c00) continue;
    const double d = fabs(av - f16_bits_to_f64((uint16_t)c));
    if (d < bestd || (d == bestd && (c & 1) == 0 && (best & 1) != 0)) {
      best = (uint16_t)c;
      bestd = d;
    }
  }
  return (uint16_t)(best | sign);
}

// lo += low fp16 half of w, hi += high half, each with one v_dot2_f32_f16
// against (1, 0) / (0, 1): the fp16 value is widened exactly and the sum is
// rounded once, as a convert-then-add would do, in half the instructions.
// w must hold finite values.
__device__ __forceinline__ void add_f16x2(uint32_t w, float& lo, float& hi) {
  typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
  const f16x2_t v = __builtin_bit_cast(f16x2_t, w);
  const f16x2_t e0 = {(_Float16)1.f, (_Float16)0.f}, e1 = {(_Float16)0.f, (_Float16)1.f};
  lo = __builtin_amdgcn_fdot2(v, e0, lo, false);
  hi = __builtin_amdgcn_fdot2(v, e1, hi, false);
}

// DPP all-reduce sum over aligned groups of L lanes (L in {1,2,4,8,16}).
// quad_perm [1,0,3,2] = 0xB1, [2,3,0,1] = 0x4E, row_half_mirror = 0x141,
// row_mirror = 0x140: each pairs every lane with a partner inside the group,
// so no source lane is ever out of range and bound_ctrl (which lets the
// compiler fold the move into a v_add_f32_dpp) changes nothing.
template <int L>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (L >= 2)
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
  if constexpr (L >= 4)
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));
  if constexpr (L >= 8)
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, true));
  if constexpr (L >= 16)
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, true));
  if constexpr (L >= 32) v += __shfl_xor(v, 16);
  if constexpr (L >= 64) v += __shfl_xor(v, 32);
  return v;
}

// max / sum over the four 16-lane groups (lanes l, l ^ 16, l ^ 32, l ^ 48)
__device__ __forceinline__ float group4_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float group4_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

}  // namespace loopvq
