// Internal device helpers shared by the libexl3 kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef _Float16 f16;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 1/sqrt(128) rounded to fp32: the normalisation of one 128-point rotation.
#define EXL3_INV_SQRT128 0.08838834764831845f

namespace exl3 {

__device__ __forceinline__ float bits_lo_f16(uint32_t w) {
  return (float)__builtin_bit_cast(f16, (uint16_t)(w & 0xFFFFu));
}
__device__ __forceinline__ float bits_hi_f16(uint32_t w) {
  return (float)__builtin_bit_cast(f16, (uint16_t)(w >> 16));
}
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  f16x2 v = {(f16)lo, (f16)hi};  // v_cvt_f16_f32: round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}

// Lane exchange inside an aligned quad of lanes via DPP quad_perm.
template <int CTRL>
__device__ __forceinline__ float quad_perm(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
#define EXL3_DPP_XOR1 0xB1  // quad_perm [1,0,3,2]
#define EXL3_DPP_XOR2 0x4E  // quad_perm [2,3,0,1]

// Unnormalised 128-point Walsh-Hadamard transform of one block held by an
// aligned quad of lanes: lane q (= lane & 3) holds elements 32q .. 32q + 31 in
// v[0..31]. Index bits 0..4 live in registers, bits 5 and 6 in the lane.
// Butterfly convention: (a, b) -> (a + b, a - b) with a the lower index, which
// yields the natural (Sylvester) order H[i][j] = (-1)^popcount(i & j).
__device__ __forceinline__ void wht128_quad(float (&v)[32], int q) {
#pragma unroll
  for (int h = 1; h < 32; h <<= 1) {
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      if ((j & h) == 0) {
        float a = v[j], b = v[j + h];
        v[j] = a + b;
        v[j + h] = a - b;
      }
    }
  }
  // bit 5: partner lane q ^ 1; lower lane keeps a + b, upper keeps a - b
  const float s1 = (q & 1) ? -1.0f : 1.0f;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    float p = quad_perm<EXL3_DPP_XOR1>(v[j]);
    v[j] = __builtin_fmaf(s1, v[j], p);
  }
  const float s2 = (q & 2) ? -1.0f : 1.0f;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    float p = quad_perm<EXL3_DPP_XOR2>(v[j]);
    v[j] = __builtin_fmaf(s2, v[j], p);
  }
}

}  // namespace exl3
