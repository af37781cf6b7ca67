// 128-point Walsh-Hadamard rotation of fp16 rows (vLLM PR #316, "Kernel
// measurements": had_r_128 on the activations before the GEMM and on its
// output after it).
//
// HBM-bound: 2 bytes read and 2 bytes written per element. 16 consecutive
// lanes own one 128-element block, one 16-byte chunk (8 elements) each, so
// every wave instruction moves 1 KB of contiguous memory. Three butterfly
// stages run in registers and four across the 16 lanes, all in fp32; the
// result is rounded once to fp16. A block lives in one wave, so in-place use
// is safe.
#include "common.h"

namespace exl3 {

template <bool PRE, bool POST>
__global__ __launch_bounds__(256) void had128_kernel(const uint16_t* in, uint16_t* out, int64_t nblocks,
                                                     int32_t blocks_per_row, const uint16_t* __restrict__ sign_pre,
                                                     const uint16_t* __restrict__ sign_post) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int q = (int)(gid & 15);
  const int64_t blk_raw = gid >> 4;
  // Lanes past the end load a valid block (whole 16-lane groups are past
  // together) and do not store.
  const int64_t blk = blk_raw < nblocks ? blk_raw : nblocks - 1;
  const int64_t col0 = (int64_t)(blk % blocks_per_row) * 128 + 8 * q;

  u32x4 d = *reinterpret_cast<const u32x4*>(in + blk * 128 + 8 * q);
  if (PRE) d ^= (*reinterpret_cast<const u32x4*>(sign_pre + col0) & 0x80008000u);  // +-1: flip the sign bit
  float v[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[2 * j] = bits_lo_f16(d[j]);
    v[2 * j + 1] = bits_hi_f16(d[j]);
  }

  wht128_16(v, q);

  u32x4 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) o[j] = pack_f16x2(v[2 * j] * EXL3_INV_SQRT128, v[2 * j + 1] * EXL3_INV_SQRT128);
  if (POST) o ^= (*reinterpret_cast<const u32x4*>(sign_post + col0) & 0x80008000u);
  if (blk_raw < nblocks) *reinterpret_cast<u32x4*>(out + blk * 128 + 8 * q) = o;
}

// The MFMA GEMMs' input operand: the same rotation of x (M x K), stored in
// fragment order for Mpad = ceil(M / 32) * 32 rows, rows past M zero, each
// fragment 1 KiB (64 lanes x 16 bytes, lane l at 16 l):
//   32-row order (the B operand of v_mfma_f32_32x32x16_f16, the dequant-GEMM):
//     block (qb, t) of 32 rows x 16 k at halves (qb * K/16 + t) * 512; lane
//     l = row % 32 + 32 * ((k % 16) / 8) holds k .. k + 7 of its row;
//   16-row order (the B operand of v_mfma_f32_16x16x32_f16, the prefill GEMM):
//     block (qb, t) of 16 rows x 32 k at halves (qb * K/32 + t) * 512; lane
//     l = row % 16 + 16 * ((k % 32) / 8) holds k .. k + 7 of its row.
// One workgroup per (32-row block, 128-column block): 16 lanes per row rotate
// as in had128_kernel, each lane two rows 16 apart (both loads in flight
// together), the results meet in LDS in fragment order, and each of the 4
// waves then stores two whole 1 KiB fragment blocks, one contiguous store
// instruction each.
template <bool PRE, bool ROWS16>
__global__ __launch_bounds__(256) void had128_frag_kernel(const uint16_t* __restrict__ in, uint16_t* __restrict__ out,
                                                          int32_t M, int32_t K, const uint16_t* __restrict__ sign_pre) {
  __shared__ u32x4 frag[8 * 64];
  const int nb = K / 128;
  const int qb = (int)(blockIdx.x / nb), b = (int)(blockIdx.x % nb);
  const int q = threadIdx.x & 15, r0 = threadIdx.x >> 4;
  const int64_t col0 = (int64_t)b * 128 + 8 * q;
  u32x4 d[2];
#pragma unroll
  for (int h = 0; h < 2; ++h)  // rows past M read row M - 1 and store zeros
    d[h] = *reinterpret_cast<const u32x4*>(in + (int64_t)min(32 * qb + r0 + 16 * h, M - 1) * K + col0);
  const u32x4 sg = PRE ? (*reinterpret_cast<const u32x4*>(sign_pre + col0) & 0x80008000u) : (u32x4){0u, 0u, 0u, 0u};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = r0 + 16 * h;
    const u32x4 x = d[h] ^ sg;
    float v[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = bits_lo_f16(x[j]);
      v[2 * j + 1] = bits_hi_f16(x[j]);
    }
    wht128_16(v, q);
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = pack_f16x2(v[2 * j] * EXL3_INV_SQRT128, v[2 * j + 1] * EXL3_INV_SQRT128);
    if (32 * qb + r >= M) o = (u32x4){0u, 0u, 0u, 0u};
    if (ROWS16)  // block (r / 16, q / 4) of this 32 x 128 piece, lane r % 16 + 16 (q % 4)
      frag[((r >> 4) * 4 + (q >> 2)) * 64 + (r & 15) + 16 * (q & 3)] = o;
    else  // block q / 2, lane r + 32 (q & 1)
      frag[(q >> 1) * 64 + r + 32 * (q & 1)] = o;
  }
  __syncthreads();
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int t = 2 * w + h;
    const int64_t blk = ROWS16 ? (int64_t)(2 * qb + (t >> 2)) * (K / 32) + 4 * b + (t & 3)
                               : (int64_t)qb * (K / 16) + 8 * b + t;
    *reinterpret_cast<u32x4*>(out + (blk * 64 + lane) * 8) = frag[t * 64 + lane];
  }
}

hipError_t launch_had128_frag(const uint16_t* in, uint16_t* out, int64_t M, int32_t K, const uint16_t* sign_pre,
                              bool rows16, hipStream_t stream) {
  const int64_t blocks = (M + 31) / 32 * (K / 128);
  if (blocks == 0) return hipSuccess;
#define EXL3_FRAG_LAUNCH(pre, r16) \
  had128_frag_kernel<pre, r16><<<(unsigned)blocks, 256, 0, stream>>>(in, out, (int32_t)M, K, sign_pre)
  if (sign_pre)
    rows16 ? EXL3_FRAG_LAUNCH(true, true) : EXL3_FRAG_LAUNCH(true, false);
  else
    rows16 ? EXL3_FRAG_LAUNCH(false, true) : EXL3_FRAG_LAUNCH(false, false);
#undef EXL3_FRAG_LAUNCH
  return hipGetLastError();
}

hipError_t launch_had128(const uint16_t* in, uint16_t* out, int64_t rows, int64_t cols, const uint16_t* sign_pre,
                         const uint16_t* sign_post, hipStream_t stream) {
  const int64_t nblocks = rows * (cols / 128);
  if (nblocks == 0) return hipSuccess;
  const int64_t threads = nblocks * 16;
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
