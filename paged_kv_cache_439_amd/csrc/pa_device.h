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
// Rotations within a row of 16 lanes (row_ror:n); ror 8 pairs lane i with i ^ 8.
constexpr int DPP_ROW_ROR1 = 0x121;
constexpr int DPP_ROW_ROR2 = 0x122;
constexpr int DPP_ROW_ROR4 = 0x124;
constexpr int DPP_ROW_ROR8 = 0x128;

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

// E4M3 quantisation, shared by the quantising store and the fused E4M3
// store + decode: element x of KV head h becomes the E4M3 code nearest to
// x / scale[h] (one IEEE fp32 division, ties to the even code), magnitudes
// saturated at 448, NaN as the NaN code 0x7F with the input's sign.

// Four fp32 values -> four E4M3 codes (byte i from y[i]).
__device__ __forceinline__ uint32_t to_e4m3x4(const float (&x)[4], float scale) {
  float y[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    y[i] = x[i] / scale;
    // saturate (comparisons with NaN are false, so NaN passes through)
    if (__builtin_fabsf(y[i]) > 448.0f) y[i] = __builtin_copysignf(448.0f, y[i]);
  }
  uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
  w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], (int)w, true);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (__builtin_isnan(y[i])) {
      const uint32_t code = 0x7Fu | (__builtin_signbit(y[i]) ? 0x80u : 0u);
      w = (w & ~(0xFFu << (8 * i))) | (code << (8 * i));
    }
  }
  return w;
}

// 16 elements of T at src -> 16 codes.
template <typename T>
__device__ __forceinline__ uint4 quantize16(const char* src, float scale) {
  float f[16];
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const uint4 v = reinterpret_cast<const uint4*>(src)[c];
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[8 * c + 2 * i] = bf16lo(w[i]);
        f[8 * c + 2 * i + 1] = bf16hi(w[i]);
      }
    }
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float4 v = reinterpret_cast<const float4*>(src)[c];
      f[4 * c] = v.x; f[4 * c + 1] = v.y; f[4 * c + 2] = v.z; f[4 * c + 3] = v.w;
    }
  }
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float x[4] = {f[4 * i], f[4 * i + 1], f[4 * i + 2], f[4 * i + 3]};
    w[i] = to_e4m3x4(x, scale);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

}  // namespace pa
