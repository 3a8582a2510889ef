// Device-side helpers shared by the HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace h3a {

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf162v __attribute__((ext_vector_type(2)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kHeadDim = 128;
constexpr int kTile = 64;
constexpr double kSqrt128 = 11.313708498984760390;               // sqrt(128)
constexpr double kInv127Sqrt128 = 1.0 / (127.0 * 11.313708498984760390);
constexpr float kInvSqrt128f = 0.088388347648318440550f;           // 1/sqrt(128)

// ---- bit-level conversions -------------------------------------------------

__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two floats -> packed fp16 pair, each rounded to nearest-even (v_cvt_pk_f16_f32).
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  float2v x = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, half2v));
}
// Two floats -> packed bf16 pair, each rounded to nearest-even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  float2v x = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf162v));
}

// Non-negative finite double -> IEEE binary16 bits, nearest-even, saturating at 65504.
__device__ __forceinline__ uint32_t f64_to_f16_rne_sat(double t) {
  if (!(t > 0.0)) return 0u;
  if (t >= 65504.0) return 0x7BFFu;
  const int e = (int)((__double_as_longlong(t) >> 52) & 0x7FF) - 1023;  // t is a normal double here
  const int qe = (e < -14 ? -14 : e) - 10;                             // exponent of one fp16 ulp
  const uint32_t m = (uint32_t)rint(ldexp(t, -qe));                     // exact scaling, one rounding
  if (e < -14) return m;                                                // subnormal (1024 -> min normal)
  return (uint32_t)((e + 15) << 10) + (m - 1024u);                      // carry into exponent is exact
}

__device__ __forceinline__ double f16_bits_to_f64(uint32_t b) {
  return (double)__builtin_bit_cast(_Float16, (uint16_t)b);
}

// ---- cross-lane moves ------------------------------------------------------

// quad_perm DPP: lane i of each quad reads lane P(i).  XOR 1 = [1,0,3,2], XOR 2 = [2,3,0,1].
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}
constexpr int kDppXor1 = 0xB1;
constexpr int kDppXor2 = 0x4E;

// Value held by lane (l ^ 32).
__device__ __forceinline__ float xor32_f32(float x) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute((int)((threadIdx.x ^ 32) << 2), __float_as_int(x)));
}

// max / sum of x over the lane pair (l, l ^ 32), with one v_permlane32_swap:
// after swapping the upper half of a with the lower half of b (a = b = x), lane
// l holds x[l ^ 32] in one of the two and x[l] in the other.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---- 128-point Walsh-Hadamard butterflies on 32 values held by one lane ----
//
// A row of 128 values is spread over 4 consecutive lanes (sub = lane & 3).
// Lane sub holds elements j = 32*k + 8*sub + e in v[8*k + e] (k = 0..3, e = 0..7):
// index bits 0-2 = e and 5-6 = k live in registers, bits 3-4 = sub across lanes.
// Each stage maps the pair (u at the index with the bit clear, w with it set)
// to (u + w, u - w): Sylvester's natural-order Hadamard, unnormalised.

__device__ __forceinline__ void fwht32_in_lane(float* v) {
#pragma unroll
  for (int m = 1; m < 8; m <<= 1)          // bits 0..2
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (!(e & m)) {
          const float u = v[8 * k + e], w = v[8 * k + e + m];
          v[8 * k + e] = u + w;
          v[8 * k + e + m] = u - w;
        }
#pragma unroll
  for (int m = 1; m < 4; m <<= 1)          // bits 5..6
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (!(k & m))
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float u = v[8 * k + e], w = v[8 * (k + m) + e];
          v[8 * k + e] = u + w;
          v[8 * (k + m) + e] = u - w;
        }
}

// Bits 3-4: exchange with lanes sub^1 and sub^2 of the same quad.
__device__ __forceinline__ void fwht32_cross_lane(float* v, int sub) {
  const float s1 = (sub & 1) ? -1.0f : 1.0f;
  const float s2 = (sub & 2) ? -1.0f : 1.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = __builtin_fmaf(v[i], s1, dpp_f32<kDppXor1>(v[i]));
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = __builtin_fmaf(v[i], s2, dpp_f32<kDppXor2>(v[i]));
}

}  // namespace h3a
