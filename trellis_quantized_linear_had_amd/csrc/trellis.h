// Device-side decode of the stand-in trellis format (format defined in exl3.h).
#pragma once

#include "common.h"

namespace exl3 {

// 2 * (x & 0xFFFF) and 2 * (x >> 16), each one SDWA VALU instruction (the
// 16-bit source select does the masking).
__device__ __forceinline__ uint32_t twice_lo16(uint32_t x, uint32_t one) {
  uint32_t r;
  asm("v_lshlrev_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:WORD_0"
      : "=v"(r)
      : "v"(one), "v"(x));
  return r;
}
__device__ __forceinline__ uint32_t twice_hi16(uint32_t x, uint32_t one) {
  uint32_t r;
  asm("v_lshlrev_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:WORD_1"
      : "=v"(r)
      : "v"(one), "v"(x));
  return r;
}

// Byte offsets (2 * state) of the 8 trellis windows that start at bit offsets
// 0, 4, ..., 28 of the 64-bit little-endian value hi:lo. One v_alignbit gives
// two windows 16 bits apart; each doubled window is one SDWA shift: 11 VALU
// instructions for 8 gather addresses.
__device__ __forceinline__ void window_offsets8(uint32_t lo, uint32_t hi, uint32_t (&off)[8]) {
  const uint32_t one = 1;
  const uint32_t a1 = __builtin_amdgcn_alignbit(hi, lo, 4);
  const uint32_t a2 = __builtin_amdgcn_alignbit(hi, lo, 8);
  const uint32_t a3 = __builtin_amdgcn_alignbit(hi, lo, 12);
  off[0] = twice_lo16(lo, one);
  off[1] = twice_lo16(a1, one);
  off[2] = twice_lo16(a2, one);
  off[3] = twice_lo16(a3, one);
  off[4] = twice_hi16(lo, one);
  off[5] = twice_hi16(a1, one);
  off[6] = twice_hi16(a2, one);
  off[7] = twice_hi16(a3, one);
}

__device__ __forceinline__ void window_states8(uint32_t lo, uint32_t hi, uint32_t (&s)[8]) {
  const uint32_t a1 = __builtin_amdgcn_alignbit(hi, lo, 4);
  const uint32_t a2 = __builtin_amdgcn_alignbit(hi, lo, 8);
  const uint32_t a3 = __builtin_amdgcn_alignbit(hi, lo, 12);
  s[0] = lo & 0xFFFFu;
  s[1] = a1 & 0xFFFFu;
  s[2] = a2 & 0xFFFFu;
  s[3] = a3 & 0xFFFFu;
  s[4] = lo >> 16;
  s[5] = a1 >> 16;
  s[6] = a2 >> 16;
  s[7] = a3 >> 16;
}

// Codebook gather from LDS: the 65536 fp16 entries sit at byte offset 2*state.
__device__ __forceinline__ uint16_t lds_cb(const uint16_t* cb_lds, uint32_t byte_off) {
  return *reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(cb_lds) + byte_off);
}

// Cooperative copy of the 128 KiB codebook from global memory into LDS.
template <int THREADS>
__device__ __forceinline__ void load_codebook(uint16_t* cb_lds, const uint16_t* __restrict__ cb) {
  const u32x4* src = reinterpret_cast<const u32x4*>(cb);
  u32x4* dst = reinterpret_cast<u32x4*>(cb_lds);
  constexpr int kChunks = 65536 * 2 / 16;
  static_assert(kChunks % THREADS == 0, "codebook copy must divide evenly");
  u32x4 tmp[kChunks / THREADS];
#pragma unroll
  for (int i = 0; i < kChunks / THREADS; ++i) tmp[i] = src[threadIdx.x + i * THREADS];
#pragma unroll
  for (int i = 0; i < kChunks / THREADS; ++i) dst[threadIdx.x + i * THREADS] = tmp[i];
}

}  // namespace exl3
