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

// RoPE on 8 rotation pairs of bf16 values: a holds x1 = x[i .. i + 7], b the
// partners x2 = x[i + D/2 .. i + D/2 + 7], c and s the cos and sin of the
// token's angles for i .. i + 7. x1' = x1 c - x2 s, x2' = x2 c + x1 s, each
// product and each sum rounded to float32 on its own (no fused multiply-add,
// whatever the unit's contraction setting), then rounded to nearest-even
// bf16. Every kernel that rotates Q or K uses this one definition, so a key
// rotated in the attention kernel has the bits of the key the page writer
// stores.
__device__ __forceinline__ void rope_bf16x8(uint4& a, uint4& b, const float* c, const float* s) {
#pragma clang fp contract(off)
  uint32_t* aw = reinterpret_cast<uint32_t*>(&a);
  uint32_t* bw = reinterpret_cast<uint32_t*>(&b);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float x1l = bf16_lo(aw[w]), x1h = bf16_hi(aw[w]);
    const float x2l = bf16_lo(bw[w]), x2h = bf16_hi(bw[w]);
    const float cl = c[2 * w], ch = c[2 * w + 1], sl = s[2 * w], sh = s[2 * w + 1];
    const float p1l = x1l * cl, q1l = x2l * sl, p2l = x2l * cl, q2l = x1l * sl;
    const float p1h = x1h * ch, q1h = x2h * sh, p2h = x2h * ch, q2h = x1h * sh;
    aw[w] = pack_bf16x2(p1l - q1l, p1h - q1h);
    bw[w] = pack_bf16x2(p2l + q2l, p2h + q2h);
  }
}

// The cos and sin of dims i .. i + 7 at table row p (float32 [max_pos, D]:
// cos in columns [0, D/2), sin in [D/2, D)), for rope_bf16x8.
__device__ __forceinline__ void rope_load8(const float* cs, int D, int p, int i, float* c,
                                           float* s) {
  const float4* cp = reinterpret_cast<const float4*>(cs + (size_t)p * D + i);
  const float4* sp = reinterpret_cast<const float4*>(cs + (size_t)p * D + D / 2 + i);
  const float4 c0 = cp[0], c1 = cp[1], s0 = sp[0], s1 = sp[1];
  c[0] = c0.x; c[1] = c0.y; c[2] = c0.z; c[3] = c0.w; c[4] = c1.x; c[5] = c1.y; c[6] = c1.z;
  c[7] = c1.w;
  s[0] = s0.x; s[1] = s0.y; s[2] = s0.z; s[3] = s0.w; s[4] = s1.x; s[5] = s1.y; s[6] = s1.z;
  s[7] = s1.w;
}

}  // namespace pa
