// 128-point Walsh-Hadamard rotation of fp16 rows (vLLM PR #316, "Kernel
// measurements": had_r_128 on the activations before the GEMM and on its
// output after it).
//
// HBM-bound: 2 bytes read and 2 bytes written per element. An aligned quad of
// lanes owns one 128-element block; each lane reads and writes 64 contiguous
// bytes. Five butterfly stages run in registers, the last two across the quad
// with DPP, all in fp32; the result is rounded once to fp16.
#include "common.h"

namespace exl3 {

template <bool PRE, bool POST>
__global__ __launch_bounds__(256) void had128_kernel(const uint16_t* in, uint16_t* out, int64_t nblocks,
                                                     int32_t blocks_per_row, const uint16_t* __restrict__ sign_pre,
                                                     const uint16_t* __restrict__ sign_post) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int q = (int)(gid & 3);
  const int64_t blk_raw = gid >> 2;
  // Lanes past the end load a valid block (whole quads are past together) and
  // do not store.
  const int64_t blk = blk_raw < nblocks ? blk_raw : nblocks - 1;
  const int64_t col0 = (int64_t)(blk % blocks_per_row) * 128 + 32 * q;

  const u32x4* src = reinterpret_cast<const u32x4*>(in + blk * 128 + 32 * q);
  u32x4 d[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) d[i] = src[i];
  if (PRE) {
    const u32x4* sp = reinterpret_cast<const u32x4*>(sign_pre + col0);
#pragma unroll
    for (int i = 0; i < 4; ++i) d[i] ^= (sp[i] & 0x80008000u);  // +-1 factor: flip the sign bit
  }
  float v[32];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[8 * i + 2 * j] = bits_lo_f16(d[i][j]);
      v[8 * i + 2 * j + 1] = bits_hi_f16(d[i][j]);
    }

  wht128_quad(v, q);

  u32x4 o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      o[i][j] = pack_f16x2(v[8 * i + 2 * j] * EXL3_INV_SQRT128, v[8 * i + 2 * j + 1] * EXL3_INV_SQRT128);
  if (POST) {
    const u32x4* sq = reinterpret_cast<const u32x4*>(sign_post + col0);
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] ^= (sq[i] & 0x80008000u);
  }
  if (blk_raw < nblocks) {
    u32x4* dst = reinterpret_cast<u32x4*>(out + blk * 128 + 32 * q);
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = o[i];
  }
}

hipError_t launch_had128(const uint16_t* in, uint16_t* out, int64_t rows, int64_t cols, const uint16_t* sign_pre,
                         const uint16_t* sign_post, hipStream_t stream) {
  const int64_t nblocks = rows * (cols / 128);
  if (nblocks == 0) return hipSuccess;
  const int64_t threads = nblocks * 4;
  const dim3 grid((unsigned)((threads + 255) / 256));
  const int32_t bpr = (int32_t)(cols / 128);
  if (sign_pre && sign_post)
    had128_kernel<true, true><<<grid, 256, 0, stream>>>(in, out, nblocks, bpr, sign_pre, sign_post);
  else if (sign_pre)
    had128_kernel<true, false><<<grid, 256, 0, stream>>>(in, out, nblocks, bpr, sign_pre, sign_post);
  else if (sign_post)
    had128_kernel<false, true><<<grid, 256, 0, stream>>>(in, out, nblocks, bpr, sign_pre, sign_post);
  else
    had128_kernel<false, false><<<grid, 256, 0, stream>>>(in, out, nblocks, bpr, sign_pre, sign_post);
  return hipGetLastError();
}

}  // namespace exl3
