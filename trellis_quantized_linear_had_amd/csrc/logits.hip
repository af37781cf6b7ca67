// Padded-width logits projection with the pad mask fused into the GEMM
// epilogue and a deterministic two-stage argmax (pegainfer PR #1046: Summary
// -- the width is rounded up to a multiple of 128 and clamped by the weight
// rows; review follow-ups -- every pad column is forced to -inf after the
// logits GEMM, inside the same owner, so selection only ever sees the
// decodable vocabulary).
//
// HBM-bound: each weight row is streamed once (2 bytes per element). A wave
// owns 64 consecutive weight rows (four 16-row MFMA tiles) over all of K and
// feeds them to v_mfma_f32_16x16x32_f16 as the A operand, with up to 16 rows of
// x as the B operand. Inside a 128-wide k chunk, MFMA step s takes the k slice
// 32 s + 8 g .. + 8 in lane group g on both operands (a permutation of k, which
// leaves the dot products unchanged), so each 16-byte load instruction reads
// 64 contiguous bytes of each of 16 rows.
#include "common.h"

namespace exl3 {

#define LG_WAVES 4

__device__ __forceinline__ void argmax_combine(float& bv, int& bi, float v, int i) {
  if (v > bv || (v == bv && i < bi)) {
    bv = v;
    bi = i;
  }
}

__global__ __launch_bounds__(64 * LG_WAVES) void logits_kernel(const uint16_t* __restrict__ x, int32_t M, int32_t K,
                                                               const uint16_t* __restrict__ w, int64_t n_valid,
                                                               int64_t n_pad, uint16_t* __restrict__ logits,
                                                               int64_t ld, bool vec_store, float* __restrict__ pv,
                                                               int32_t* __restrict__ pi, int64_t n_items, int32_t m0) {
  const int64_t item = (int64_t)blockIdx.x * LG_WAVES + (threadIdx.x >> 6);
  if (item >= n_items) return;  // whole wave; no workgroup barriers below
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, pl = lane & 15;
  const int64_t p0 = item * 64;
  const int q = m0 + pl;

  f32x4 acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) acc[t] = (f32x4){0.f, 0.f, 0.f, 0.f};

  const uint16_t* wrow[4];
  bool wok[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int64_t row = p0 + 16 * t + pl;
    wok[t] = row < n_pad;
    wrow[t] = w + (wok[t] ? row : 0) * (int64_t)K + 8 * g;
  }
  const bool qok = q < M;
  const uint16_t* xrow = x + (int64_t)(qok ? q : 0) * K + 8 * g;

  for (int kc = 0; kc < K; kc += 128) {
    u32x4 av[4][4], bv[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        av[t][s] = wok[t] ? *reinterpret_cast<const u32x4*>(wrow[t] + kc + 32 * s) : (u32x4){0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < 4; ++s)
      bv[s] = qok ? *reinterpret_cast<const u32x4*>(xrow + kc + 32 * s) : (u32x4){0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int t = 0; t < 4; ++t)
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, av[t][s]),
                                                        __builtin_bit_cast(f16x8, bv[s]), acc[t], 0, 0, 0);
  }

  // Epilogue: lane holds D[p = p0 + 16t + 4g + r][q]; round to fp16, mask the
  // pad columns, store, and keep the first maximum.
  float best = -__builtin_inff();
  int besti = 0x7FFFFFFF;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int64_t pb = p0 + 16 * t + 4 * g;
    uint16_t h[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t p = pb + r;
      const f16 v = (f16)acc[t][r];
      h[r] = (p < n_valid) ? __builtin_bit_cast(uint16_t, v) : (uint16_t)0xFC00;
      if (p < n_pad) argmax_combine(best, besti, (float)__builtin_bit_cast(f16, h[r]), (int)p);
    }
    if (qok) {
      uint16_t* dst = logits + (int64_t)q * ld + pb;
      if (vec_store && pb + 3 < n_pad) {
        u32x2 o = {(uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16)};
        *reinterpret_cast<u32x2*>(dst) = o;
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (pb + r < n_pad) dst[r] = h[r];
      }
    }
  }
  // lanes pl, pl+16, pl+32, pl+48 hold the same output row q
#pragma unroll
  for (int o = 16; o <= 32; o <<= 1) {
    const float v2 = __shfl_xor(best, o);
    const int i2 = __shfl_xor(besti, o);
    argmax_combine(best, besti, v2, i2);
  }
  if (g == 0 && qok) {
    pv[item * M + q] = best;
    pi[item * M + q] = besti;
  }
}

// argmax[q] over the per-wave (max, first index) pairs; any combination order
// gives the same (largest value, smallest index) pair.
__global__ __launch_bounds__(256) void argmax_final_kernel(const float* __restrict__ pv, const int32_t* __restrict__ pi,
                                                           int64_t n_items, int32_t M, int64_t* __restrict__ out) {
  __shared__ float sv[256];
  __shared__ int si[256];
  const int q = blockIdx.x;
  float best = -__builtin_inff();
  int besti = 0x7FFFFFFF;
  for (int64_t it = threadIdx.x; it < n_items; it += 256) argmax_combine(best, besti, pv[it * M + q], pi[it * M + q]);
  sv[threadIdx.x] = best;
  si[threadIdx.x] = besti;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) {
      float b = sv[threadIdx.x];
      int bi = si[threadIdx.x];
      argmax_combine(b, bi, sv[threadIdx.x + s], si[threadIdx.x + s]);
      sv[threadIdx.x] = b;
      si[threadIdx.x] = bi;
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) out[q] = si[0];
}

int64_t logits_items(int64_t n_pad) { return (n_pad + 63) / 64; }

hipError_t launch_logits(const uint16_t* x, int32_t M, int32_t K, const uint16_t* w, int64_t n_valid, int64_t n_pad,
                         uint16_t* logits, int64_t ld, int64_t* argmax, float* pv, int32_t* pi, hipStream_t stream) {
  const int64_t n_items = logits_items(n_pad);
  const bool vec = (ld % 4) == 0 && ((uintptr_t)logits % 8) == 0;
  const unsigned grid = (unsigned)((n_items + LG_WAVES - 1) / LG_WAVES);
  for (int32_t m0 = 0; m0 < M; m0 += 16) {
    logits_kernel<<<grid, 64 * LG_WAVES, 0, stream>>>(x, M, K, w, n_valid, n_pad, logits, ld, vec, pv, pi, n_items,
                                                      m0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  argmax_final_kernel<<<M, 256, 0, stream>>>(pv, pi, n_items, M, argmax);
  return hipGetLastError();
}

}  // namespace exl3
