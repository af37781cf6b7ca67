// Pad mask and argmax of the quantized output head (the padded-logits rule
// of pegainfer PR #1046, Summary and review follow-ups, applied to a trellis
// layer's first n_pad columns): a separate pass over logits that the layer's
// kernels have already written.
#include <algorithm>

#include "common.h"

namespace exl3 {

hipError_t launch_argmax_final(const int32_t* pk, const int32_t* pi, int64_t n_items, int64_t M, int64_t* out,
                               hipStream_t stream);

// Pad mask and argmax over logits that another kernel has already written
// (the quantized head: the layer's first n_pad columns), in two stages like
// the projection's. Stage one: a workgroup per (row, MA_COLS-column piece);
// each thread takes two 16-byte chunks (n_pad and ld are multiples of 8, so a
// chunk never crosses the row end), rewrites every chunk holding columns at
// or past n_valid with those set to -inf, and the workgroup reduces its
// (largest value, smallest index) pair over the piece, pads included. Stage
// two is the logits projection's per-row reduce over the pieces.
#define MA_THREADS 256
#define MA_COLS (MA_THREADS * 16)
__global__ __launch_bounds__(MA_THREADS) void head_mask_argmax_kernel(uint16_t* __restrict__ logits, int64_t ld,
                                                                      int64_t n_valid, int64_t n_pad,
                                                                      int64_t n_items, int32_t* __restrict__ pk,
                                                                      int32_t* __restrict__ pi) {
  __shared__ int sv[MA_THREADS / 64];
  __shared__ int si[MA_THREADS / 64];
  const int64_t q = blockIdx.x / n_items, item = blockIdx.x % n_items;
  uint16_t* row = logits + q * ld;
  int best = EXL3_KEY_NONE;
  int besti = 0x7FFFFFFF;
  u32x4 v[2];
  int64_t c[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    c[h] = item * MA_COLS + h * (MA_COLS / 2) + threadIdx.x * 8;
    if (c[h] < n_pad) v[h] = *reinterpret_cast<const u32x4*>(row + c[h]);
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if (c[h] >= n_pad) continue;
    if (c[h] + 8 > n_valid) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (c[h] + j >= n_valid) {
          const int sh = 16 * (j & 1);
          v[h][j >> 1] = (v[h][j >> 1] & ~(0xFFFFu << sh)) | (0xFC00u << sh);
        }
      *reinterpret_cast<u32x4*>(row + c[h]) = v[h];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint16_t e = (uint16_t)(v[h][j >> 1] >> (16 * (j & 1)));
      argmax_combine(best, besti, argmax_key(e), (int)(c[h] + j));
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const int ov = __shfl_xor(best, off);
    const int oi = __shfl_xor(besti, off);
    argmax_combine(best, besti, ov, oi);
  }
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sv[wave] = best;
    si[wave] = besti;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < MA_THREADS / 64; ++w) argmax_combine(best, besti, sv[w], si[w]);
    pk[q * n_items + item] = best;
    pi[q * n_items + item] = besti;
  }
}

int64_t head_argmax_items(int64_t n_pad) { return (n_pad + MA_COLS - 1) / MA_COLS; }

hipError_t launch_head_mask_argmax(uint16_t* logits, int64_t ld, int64_t M, int64_t n_valid, int64_t n_pad,
                                   int64_t* argmax, int32_t* pk, int32_t* pi, hipStream_t stream) {
  const int64_t n_items = head_argmax_items(n_pad);
  // rows per launch keep every grid well below 2^32 work-items
  const int64_t rows = std::max<int64_t>(1, ((int64_t)1 << 22) / n_items);
  for (int64_t m0 = 0; m0 < M; m0 += rows) {
    const int64_t mr = std::min(rows, M - m0);
    head_mask_argmax_kernel<<<(unsigned)(mr * n_items), MA_THREADS, 0, stream>>>(
        logits + m0 * ld, ld, n_valid, n_pad, n_items, pk + m0 * n_items, pi + m0 * n_items);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_argmax_final(pk + m0 * n_items, pi + m0 * n_items, n_items, mr, argmax + m0, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace exl3
