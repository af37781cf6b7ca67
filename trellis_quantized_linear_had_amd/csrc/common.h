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

// Buffer resource descriptor over [p, p + bytes): raw (untyped) 32-bit loads
// with a wave-uniform scalar offset and a per-lane 32-bit offset. Third word:
// the raw-buffer data format for gfx9-family parts.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint32_t buffer_load_u32(__amdgpu_buffer_rsrc_t r, uint32_t voff_bytes, uint32_t soff_bytes) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff_bytes, soff_bytes, 0);
}

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

// Lane exchange by one DPP move; CTRL is the DPP control word (quad_perm,
// row_mirror, row_half_mirror, ...), all rows and banks enabled.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
#define EXL3_DPP_XOR1 0xB1  // quad_perm [1,0,3,2]
#define EXL3_DPP_XOR2 0x4E  // quad_perm [2,3,0,1]
#define EXL3_DPP_REV4 0x1B  // quad_perm [3,2,1,0]: lane ^ 3
#define EXL3_DPP_HALF_MIRROR 0x141  // lane ^ 7 within 8 lanes
#define EXL3_DPP_MIRROR 0x140       // lane ^ 15 within 16 lanes
#define EXL3_DPP_PAIR_LO 0x50       // quad_perm [0,0,1,1]
#define EXL3_DPP_PAIR_HI 0xFA       // quad_perm [2,2,3,3]

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_mov_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}

// Value of lane ^ 4 and lane ^ 8 (within 16 lanes) by two DPP moves each,
// on the VALU rather than the LDS crossbar: (l ^ 7) ^ 3 = l ^ 4 and
// (l ^ 15) ^ 7 = l ^ 8.
__device__ __forceinline__ float lane_xor4(float v) {
  return dpp_mov<EXL3_DPP_REV4>(dpp_mov<EXL3_DPP_HALF_MIRROR>(v));
}
__device__ __forceinline__ float lane_xor8(float v) {
  return dpp_mov<EXL3_DPP_HALF_MIRROR>(dpp_mov<EXL3_DPP_MIRROR>(v));
}

// Unnormalised 128-point Walsh-Hadamard transform of one block held by 16
// consecutive lanes: lane q (= lane & 15) holds elements 8q .. 8q + 7 in
// v[0..7]. Index bits 0..2 live in registers, bits 3..6 in the lane (all four
// partners q ^ 1, q ^ 2, q ^ 4, q ^ 8 by DPP). Butterfly convention:
// (a, b) -> (a + b, a - b) with a the lower index, which yields the natural
// (Sylvester) order H[i][j] = (-1)^popcount(i & j).
__device__ __forceinline__ void wht128_16(float (&v)[8], int q) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if ((j & h) == 0) {
        float a = v[j], b = v[j + h];
        v[j] = a + b;
        v[j + h] = a - b;
      }
    }
  }
  const float s1 = (q & 1) ? -1.0f : 1.0f, s2 = (q & 2) ? -1.0f : 1.0f;
  const float s4 = (q & 4) ? -1.0f : 1.0f, s8 = (q & 8) ? -1.0f : 1.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = __builtin_fmaf(s1, v[j], dpp_mov<EXL3_DPP_XOR1>(v[j]));
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = __builtin_fmaf(s2, v[j], dpp_mov<EXL3_DPP_XOR2>(v[j]));
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = __builtin_fmaf(s4, v[j], lane_xor4(v[j]));
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = __builtin_fmaf(s8, v[j], lane_xor8(v[j]));
}

// Order key of an fp16 logit for the argmax, which follows NumPy's and
// torch's rule: a NaN ranks above every number (all NaNs tie, so the first
// NaN wins), -0 ties with +0, and otherwise keys follow the values. Integer
// compares on these keys replace float compares, which would never select a
// NaN.
#define EXL3_KEY_NONE (-0x7FFFFFFF - 1)  // below every key: no candidate yet
__device__ __forceinline__ int argmax_key(uint16_t h) {
  const int mag = h & 0x7FFF;
  if (mag > 0x7C00) return 0x7C01;
  return (h & 0x8000) ? -mag : mag;
}

// (largest key, smallest index): any combination order gives the same pair.
__device__ __forceinline__ void argmax_combine(int& bk, int& bi, int k, int i) {
  if (k > bk || (k == bk && i < bi)) {
    bk = k;
    bi = i;
  }
}

}  // namespace exl3
