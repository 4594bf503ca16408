// Device helpers shared by the gfx950 kernels of libpagedattn.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// A finite stand-in for "no logit seen yet": exp2(NEG_BIG - x) is 0 for any
// real logit x, and exp2(NEG_BIG - NEG_BIG) is 1, so empty softmax states
// merge without producing NaN.
constexpr float NEG_BIG = -1.0e30f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Lane permutations within a row of 16 lanes (DPP). Used as butterflies for
// all-reduce sums: xor 1, xor 2, then the half-row and full-row mirrors,
// which pair every lane of one half with a lane of the other half.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
constexpr int DPP_XOR1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141; // lane i <-> 7-i within 8
constexpr int DPP_MIRROR = 0x140;      // lane i <-> 15-i within 16

// Sum over aligned groups of N consecutive lanes (N in {1,2,4,8,16,32});
// every lane of a group receives the group's total.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (N >= 2) v += dpp_f32<DPP_XOR1>(v);
  if constexpr (N >= 4) v += dpp_f32<DPP_XOR2>(v);
  if constexpr (N >= 8) v += dpp_f32<DPP_HALF_MIRROR>(v);
  if constexpr (N >= 16) v += dpp_f32<DPP_MIRROR>(v);
  if constexpr (N >= 32) v += __shfl_xor(v, 16);
  return v;
}

// bf16 <-> fp32. A bf16 is the high half of an fp32, so widening is a shift.
__device__ __forceinline__ float bf16lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

// Round-to-nearest-even fp32 -> bf16 bits (the hardware conversion).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}
// The same rounding of two values with one v_cvt_pk_bf16_f32.
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

__device__ __forceinline__ int clamp_block(int b, int num_blocks) {
  return min(max(b, 0), num_blocks - 1);
}

}  // namespace pa
