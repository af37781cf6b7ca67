// Output stage shared by the MFMA kernels that compute the transposed
// product D[p][q] (p = output column, q = input row) in the accumulator
// layouts of v_mfma_f32_32x32x16_f16 and v_mfma_f32_16x16x32_f16: the
// 128-point output rotation along p, the sign vector, the 1/sqrt(128) scaling
// and the fp16 store of y[q][p].
#pragma once

#include "common.h"

namespace exl3 {

// The butterfly between lanes M apart (M = 16 or 32) without the LDS: a
// permlane swap of the value with itself leaves, in every lane of a pair of
// M-lane rows, the lower row's value in its first result and the upper row's
// in its second. With s = +1 in the lower row and -1 in the upper one this
// gives lower + upper and lower - upper, the same roundings as adding the
// partner's value from a shuffle. Every lane of the wave must be active.
template <int M>
__device__ __forceinline__ float xor_butterfly(float v, float s) {
  static_assert(M == 16 || M == 32, "rows of 16 or 32 lanes");
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  uint32_t lo, hi;
  if constexpr (M == 16) {
    const auto w = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    lo = w[0];
    hi = w[1];
  } else {
    const auto w = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    lo = w[0];
    hi = w[1];
  }
  return __builtin_fmaf(s, __builtin_bit_cast(float, hi), __builtin_bit_cast(float, lo));
}

// Output rotation + signs + fp16 store of one 128 (p) x 32 (q) block of a
// wave. a[i][r] holds D[p][q] with (inside the 128-row rotation block)
// p = 32 i + 8 (r >> 2) + 4 lhalf + (r & 3), q = q0 + lrow. Index bits of p:
// 0,1 <- r&3; 2 <- lhalf; 3,4 <- r>>2; 5,6 <- i. Six stages in registers, one
// across lanes 32 apart.
__device__ __forceinline__ void rotate_store_block(f32x16 (&a)[4], int lane, int pw, int q0, int P, int Q,
                                                   uint16_t* __restrict__ y, int64_t ldy, int32_t n0,
                                                   const uint16_t* __restrict__ sign_n) {
  const int lrow = lane & 31, lhalf = lane >> 5;
  // The 16 sign words go out before the butterflies and are used after them:
  // one memory round trip, under the arithmetic, and no wait between the
  // stores. Without signs, row 0 of y (in bounds, then masked off) is read.
  u32x2 sg[4][4];
  const uint32_t smask = sign_n ? 0x80008000u : 0u;
  if (pw < P) {  // uniform over the wave
    const uint16_t* sp = (sign_n ? sign_n : y) + n0 + pw;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) sg[i][g] = *reinterpret_cast<const u32x2*>(sp + 32 * i + 8 * g + 4 * lhalf);
  }
#pragma unroll
  for (int h = 1; h <= 8; h <<= 1) {  // register bits r&1, r&2, r&4, r&8
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if ((r & h) == 0) {
          const float u = a[i][r], v = a[i][r + h];
          a[i][r] = u + v;
          a[i][r + h] = u - v;
        }
  }
#pragma unroll
  for (int h = 1; h <= 2; h <<= 1) {  // register bits of i
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if ((i & h) == 0)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float u = a[i][r], v = a[i + h][r];
          a[i][r] = u + v;
          a[i + h][r] = u - v;
        }
  }
  const float s = lhalf ? -1.f : 1.f;  // lane bit: partner 32 lanes away
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) a[i][r] = xor_butterfly<32>(a[i][r], s);
  if (pw >= P) return;
  const int q = q0 + lrow;
  if (q >= Q) return;
  uint16_t* yrow = y + (int64_t)q * ldy + n0 + pw;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int p = 32 * i + 8 * g + 4 * lhalf;
      u32x2 o;
      o[0] = pack_f16x2(a[i][4 * g] * EXL3_INV_SQRT128, a[i][4 * g + 1] * EXL3_INV_SQRT128);
      o[1] = pack_f16x2(a[i][4 * g + 2] * EXL3_INV_SQRT128, a[i][4 * g + 3] * EXL3_INV_SQRT128);
      o ^= sg[i][g] & smask;
      *reinterpret_cast<u32x2*>(yrow + p) = o;
    }
}

// The same output stage for a wave holding v_mfma_f32_16x16x32_f16
// accumulators of one 128 (p) x 16 (q) block: a[i][r] = D[p][q] with (inside
// the 128-row rotation block) p = 16 i + 4 (lane >> 4) + r, q = q0 + (lane & 15).
// Index bits of p: 0,1 <- r; 2,3 <- lane bits 4,5; 4,5,6 <- i. Five stages in
// registers, two across lanes 16 and 32 apart.
__device__ __forceinline__ void rotate_store_block16(f32x4 (&a)[8], int lane, int pw, int q0, int P, int Q,
                                                     uint16_t* __restrict__ y, int64_t ldy, int32_t n0,
                                                     const uint16_t* __restrict__ sign_n) {
  const int lq = lane & 15, lg = lane >> 4;
  // the 8 sign words go out before the butterflies (one memory round trip);
  // without signs, row 0 of y (in bounds, then masked off) is read
  u32x2 sg[8];
  const uint32_t smask = sign_n ? 0x80008000u : 0u;
  if (pw < P) {  // uniform over the wave
    const uint16_t* sp = (sign_n ? sign_n : y) + n0 + pw;
#pragma unroll
    for (int i = 0; i < 8; ++i) sg[i] = *reinterpret_cast<const u32x2*>(sp + 16 * i + 4 * lg);
  }
#pragma unroll
  for (int h = 1; h <= 2; h <<= 1)  // register bits r&1, r&2
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if ((r & h) == 0) {
          const float u = a[i][r], v = a[i][r + h];
          a[i][r] = u + v;
          a[i][r + h] = u - v;
        }
#pragma unroll
  for (int h = 1; h <= 4; h <<= 1)  // register bits of i
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if ((i & h) == 0)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float u = a[i][r], v = a[i + h][r];
          a[i][r] = u + v;
          a[i + h][r] = u - v;
        }
  {  // lane bits 4, 5: the partner 16, then 32 lanes away
    const float s16 = (lane & 16) ? -1.f : 1.f, s32 = (lane & 32) ? -1.f : 1.f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) a[i][r] = xor_butterfly<16>(a[i][r], s16);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) a[i][r] = xor_butterfly<32>(a[i][r], s32);
  }
  if (pw >= P) return;
  const int q = q0 + lq;
  if (q >= Q) return;
  uint16_t* yrow = y + (int64_t)q * ldy + n0 + pw;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    u32x2 o;
    o[0] = pack_f16x2(a[i][0] * EXL3_INV_SQRT128, a[i][1] * EXL3_INV_SQRT128);
    o[1] = pack_f16x2(a[i][2] * EXL3_INV_SQRT128, a[i][3] * EXL3_INV_SQRT128);
    o ^= sg[i] & smask;
    *reinterpret_cast<u32x2*>(yrow + 16 * i + 4 * lg) = o;
  }
}

// The same output stage split for a block whose two 64-row halves sit in two
// waves (the dequant-GEMM): each wave runs the six stages inside its half on
// its tiles t[0], t[1] (p = 32 f + 8 (r >> 2) + 4 lhalf + (r & 3): register
// bits 0, 1, 3, 4, the tile bit 5, the lane bit 2) ...
__device__ __forceinline__ void wht64_half(f32x16 (&t)[2], int lane) {
#pragma unroll
  for (int h = 1; h <= 8; h <<= 1)
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if ((r & h) == 0) {
          const float u = t[f][r], v = t[f][r + h];
          t[f][r] = u + v;
          t[f][r + h] = u - v;
        }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const float u = t[0][r], v = t[1][r];
    t[0][r] = u + v;
    t[1][r] = u - v;
  }
  const float s = (lane >> 5) ? -1.f : 1.f;
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int r = 0; r < 16; ++r) t[f][r] = xor_butterfly<32>(t[f][r], s);
}

// ... and the wave that stores a block combines the halves (bit 6: lo + hi
// for tile f, lo - hi for tile 2 + f), applies the signs and 1/sqrt(128) and
// stores fp16 y[q][n0 + pw + p], one tile index f at a time.
__device__ __forceinline__ void store_halves_tile(const f32x16& lo, const f32x16& hi, int f, int lane, int pw, int q0,
                                                  int P, int Q, uint16_t* __restrict__ y, int64_t ldy, int32_t n0,
                                                  const uint16_t* __restrict__ sign_n) {
  const int lrow = lane & 31, lhalf = lane >> 5;
  if (pw >= P) return;
  const int q = q0 + lrow;
  if (q >= Q) return;
  const uint32_t smask = sign_n ? 0x80008000u : 0u;
  const uint16_t* sp = (sign_n ? sign_n : y) + n0 + pw;
  uint16_t* yrow = y + (int64_t)q * ldy + n0 + pw;
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int p = 32 * (f + 2 * half) + 8 * g + 4 * lhalf;
      const u32x2 sg = *reinterpret_cast<const u32x2*>(sp + p);
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = half ? lo[4 * g + e] - hi[4 * g + e] : lo[4 * g + e] + hi[4 * g + e];
      u32x2 o;
      o[0] = pack_f16x2(v[0] * EXL3_INV_SQRT128, v[1] * EXL3_INV_SQRT128);
      o[1] = pack_f16x2(v[2] * EXL3_INV_SQRT128, v[3] * EXL3_INV_SQRT128);
      o ^= sg & smask;
      *reinterpret_cast<u32x2*>(yrow + p) = o;
    }
}

}  // namespace exl3
