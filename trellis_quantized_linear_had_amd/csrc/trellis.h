// Device-side decode of the stand-in trellis format (format defined in exl3.h):
// b bits per weight, 16x16 tiles of 8b little-endian words, state(i) = the
// 16-bit window at bit b*i of the tile, wrapping at its 256b bits.
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

// At 4 bits a 32-k MFMA step's B-fragment lanes hold word 2 i + (r & 1) of
// their k-tile's 32 code words in lane 16 r + i (rows r = 0, 1 of the first
// k-tile, 2, 3 of the second). The word after a lane's own sits in the same
// lane of the paired row (rows 0, 2) or one lane further in it, lane 15
// wrapping to word 0 (rows 1, 3): one row swap and one in-row rotation, with
// every lane active.
__device__ __forceinline__ uint32_t next_tile_word(uint32_t w) {
  const auto sw = __builtin_amdgcn_permlane16_swap(w, w, false, false);
  // rows 1, 3 take sw[0] rotated one lane down (row_ror:15); rows 0, 2 keep sw[1]
  return __builtin_amdgcn_update_dpp(sw[1], sw[0], 0x12F, 0xA, 0xF, false);
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

// Windows of NS consecutive steps at any width. A lane whose first window
// starts at bit `start` of its tile holds the NW words from word start / 32
// on (mod the tile's 8 BITS words): w[j] = tile[(start / 32 + j) % (8 BITS)],
// and off = start % 32. One funnel shift per word drops the offset; after it
// window r starts at bit r * BITS, a compile-time position, so each window is
// at most one v_alignbit plus one SDWA shift.
template <int BITS>
struct TrellisWidth {
  static_assert(BITS >= 1 && BITS <= 8, "1..8 bits per weight");
  static constexpr int kTileWords = 8 * BITS;
  static constexpr int kTileBytes = 32 * BITS;
  // largest start % 32 of a window run that begins at a step that is a
  // multiple of `step_align` (16: a tile column; 8: half a column)
  static constexpr int off_max(int step_align) {
    return (step_align * BITS) % 32 == 0 ? 0 : (step_align * BITS) % 16 == 0 ? 16 : (step_align * BITS) % 8 == 0 ? 24 : 31;
  }
  // words a lane loads for NS windows whose first step is a multiple of step_align
  static constexpr int words(int ns, int step_align) { return (off_max(step_align) + BITS * (ns - 1) + 16 + 31) / 32; }
};

template <int BITS, int NS, int NW>
__device__ __forceinline__ void window_offsets_any(const uint32_t (&w)[NW], uint32_t off, uint32_t (&out)[NS]) {
  constexpr int NA = (BITS * (NS - 1) + 16 + 31) / 32;  // words after the shift
  static_assert(NA <= NW, "too few words for the windows");
  const uint32_t one = 1;
  uint32_t a[NA + 1];
#pragma unroll
  for (int j = 0; j < NA; ++j) a[j] = __builtin_amdgcn_alignbit(j + 1 < NW ? w[j + 1] : 0u, w[j], off);
  a[NA] = 0;
#pragma unroll
  for (int r = 0; r < NS; ++r) {
    const int pos = r * BITS, idx = pos >> 5, sh = pos & 31;
    if (sh == 0)
      out[r] = twice_lo16(a[idx], one);
    else if (sh == 16)
      out[r] = twice_hi16(a[idx], one);
    else
      out[r] = twice_lo16(__builtin_amdgcn_alignbit(a[idx + 1], a[idx], sh), one);
  }
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
