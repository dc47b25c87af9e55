// Device helpers shared by the gfx950 kernels of libpa: bf16 bit handling,
// 16-byte vector loads, and cross-lane sums with DPP.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr float kLog2e = 1.4426950408889634f;
// Running-max start value: finite, so exp2(m_old - m_new) is 0 (not NaN) on the
// first block, and far below any real logit.
constexpr float kNegBig = -1.0e30f;

// ---- bf16 <-> f32 (bf16 = high half of an IEEE binary32) ----
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Round to nearest, ties to even. NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return ((u >> 16) | 0x40u) & 0xFFFFu;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

// Element type tags.
struct F32 {
  typedef float storage;
  static constexpr int kBytes = 4;
};
struct BF16 {
  typedef uint16_t storage;
  static constexpr int kBytes = 2;
};

// ---- cross-lane ----
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of N consecutive lanes (N = 1, 2, 4, 8, 16, 32, 64);
// every lane of a group ends with the same bits (each step adds a commutative
// pair, so lane order never changes the rounding).
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp_f<0xB1>(x);   // quad_perm [1,0,3,2]: partner lane ^ 1
  if constexpr (N >= 4) x += dpp_f<0x4E>(x);   // quad_perm [2,3,0,1]: partner lane ^ 2
  if constexpr (N >= 8) x += dpp_f<0x141>(x);  // row_half_mirror: other quad of the 8
  if constexpr (N >= 16) x += dpp_f<0x140>(x); // row_mirror: other half of the 16-lane row
  if constexpr (N >= 32) x += __shfl_xor(x, 16);
  if constexpr (N >= 64) x += __shfl_xor(x, 32);
  return x;
}

template <int N>
__device__ __forceinline__ float group_max(float x) {
  if constexpr (N >= 2) x = fmaxf(x, dpp_f<0xB1>(x));
  if constexpr (N >= 4) x = fmaxf(x, dpp_f<0x4E>(x));
  if constexpr (N >= 8) x = fmaxf(x, dpp_f<0x141>(x));
  if constexpr (N >= 16) x = fmaxf(x, dpp_f<0x140>(x));
  if constexpr (N >= 32) x = fmaxf(x, __shfl_xor(x, 16));
  if constexpr (N >= 64) x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---- bf16 vectors for v_dot2 / v_cvt_pk / MFMA operands ----
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __bf16 bf16x2e_t __attribute__((ext_vector_type(2)));

// acc + a.lo * b.lo + a.hi * b.hi (bf16 pairs, float32 accumulation)
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

}  // namespace pa
