// Padded-width logits projection with the pad mask fused into the GEMM
// epilogue and a deterministic two-stage argmax (pegainfer PR #1046: Summary
// -- the width is rounded up to a multiple of 128 and clamped by the weight
// rows; review follow-ups -- every pad column is forced to -inf after the
// logits GEMM, inside the same owner, so selection only ever sees the
// decodable vocabulary).
//
// HBM-bound: each weight row is streamed once (2 bytes per element). A wave
// owns 128 consecutive weight rows (eight 16-row MFMA tiles) over all of K and
// feeds them to v_mfma_f32_16x16x32_f16 as the A operand, with 16 rows of x as
// the B operand. Inside a 64-wide k chunk, MFMA step s takes the k slice
// 32 s + 8 g .. + 8 in lane group g on both operands (a permutation of k, which
// leaves the dot products unchanged), so each 16-byte load instruction reads
// 64 contiguous bytes of each of 16 weight rows. A pre-pass stores x in that
// fragment order (rows past M zero), so each B-fragment load reads 1 KiB of
// contiguous memory instead of 16 rows 2K bytes apart, which measured ~40 us
// slower per call at M = 16 (the row-strided lines crowd a few L2 channels).
// The loads of the next chunk are issued before the MFMAs of the current one.
#include "common.h"
#include "marks.h"

namespace exl3 {

#define LG_WAVES 4
#define LG_ROWS 128             // weight rows per wave
#define LG_TILES (LG_ROWS / 16)
#define LG_KC 64                // k per chunk
#define LG_STEPS (LG_KC / 32)

// x (M x K) -> xp[mg][j][g][q][0..8) = x[16 mg + q][32 j + 8 g + 0..8], zero
// for rows past M: the B fragment of lane (g, q) at k-step j, for row group
// mg, is 16 contiguous bytes and a wave's 64 fragments are 1 KiB.
__global__ __launch_bounds__(256) void logits_xperm_kernel(const uint16_t* __restrict__ x, int32_t M, int32_t K,
                                                           uint16_t* __restrict__ xp, int64_t nchunks) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;  // 16-byte chunk of xp
  if (c >= nchunks) return;
  const int q = (int)(c & 15), g = (int)((c >> 4) & 3);
  const int64_t jm = c >> 6;  // mg * (K / 32) + j
  const int64_t mg = jm / (K / 32), j = jm - mg * (K / 32);
  const int64_t row = mg * 16 + q;
  u32x4 v = {0, 0, 0, 0};
  if (row < M) v = *reinterpret_cast<const u32x4*>(x + row * K + 32 * j + 8 * g);
  *reinterpret_cast<u32x4*>(xp + c * 8) = v;
}

// Loads one LG_KC-wide chunk: LG_TILES x LG_STEPS weight fragments and the
// LG_STEPS x fragments.
__device__ __forceinline__ void logits_load_chunk(const uint16_t* const (&wrow)[LG_TILES], const uint16_t* xfrag,
                                                  int kc, u32x4 (&av)[LG_TILES][LG_STEPS], u32x4 (&bv)[LG_STEPS]) {
#pragma unroll
  for (int t = 0; t < LG_TILES; ++t)
#pragma unroll
    for (int s = 0; s < LG_STEPS; ++s) av[t][s] = *reinterpret_cast<const u32x4*>(wrow[t] + kc + 32 * s);
#pragma unroll
  for (int s = 0; s < LG_STEPS; ++s) bv[s] = *reinterpret_cast<const u32x4*>(xfrag + (int64_t)(kc / 32 + s) * 64 * 8);
}

__device__ __forceinline__ void logits_mfma_chunk(const u32x4 (&av)[LG_TILES][LG_STEPS], const u32x4 (&bv)[LG_STEPS],
                                                  f32x4 (&acc)[LG_TILES]) {
#pragma unroll
  for (int s = 0; s < LG_STEPS; ++s)
#pragma unroll
    for (int t = 0; t < LG_TILES; ++t)
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, av[t][s]),
                                                      __builtin_bit_cast(f16x8, bv[s]), acc[t], 0, 0, 0);
}

__global__ __launch_bounds__(64 * LG_WAVES) void logits_kernel(const uint16_t* __restrict__ xp, int32_t M, int32_t K,
                                                               const uint16_t* __restrict__ w, int64_t n_valid,
                                                               int64_t n_pad, uint16_t* __restrict__ logits,
                                                               int64_t ld, bool vec_store, int32_t* __restrict__ pk,
                                                               int32_t* __restrict__ pi, int64_t n_items, int32_t m0) {
  const int64_t item = (int64_t)blockIdx.x * LG_WAVES + (threadIdx.x >> 6);
  if (item >= n_items) return;  // whole wave; no workgroup barriers below
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, pl = lane & 15;
  const int64_t p0 = item * LG_ROWS;
  const int q = m0 + pl;

  f32x4 acc[LG_TILES];
#pragma unroll
  for (int t = 0; t < LG_TILES; ++t) acc[t] = (f32x4){0.f, 0.f, 0.f, 0.f};

  // Rows past the padded width read row 0 instead (valid memory, no branch
  // in the loop); their sums are never stored or ranked.
  const uint16_t* wrow[LG_TILES];
#pragma unroll
  for (int t = 0; t < LG_TILES; ++t) {
    const int64_t row = p0 + 16 * t + pl;
    wrow[t] = w + (row < n_pad ? row : 0) * (int64_t)K + 8 * g;
  }
  const uint16_t* xfrag = xp + ((int64_t)(m0 / 16) * (K / 32) * 64 + lane) * 8;

  // Two chunk buffers: chunk c + 1 is in flight while the MFMAs of chunk c
  // run (K is a multiple of 128, so chunks come in pairs).
  u32x4 av0[LG_TILES][LG_STEPS], bv0[LG_STEPS], av1[LG_TILES][LG_STEPS], bv1[LG_STEPS];
  logits_load_chunk(wrow, xfrag, 0, av0, bv0);
  for (int kc = 0; kc < K; kc += 2 * LG_KC) {
    logits_load_chunk(wrow, xfrag, kc + LG_KC, av1, bv1);
    __builtin_amdgcn_sched_barrier(0);
    logits_mfma_chunk(av0, bv0, acc);
    if (kc + 2 * LG_KC < K) logits_load_chunk(wrow, xfrag, kc + 2 * LG_KC, av0, bv0);  // uniform
    __builtin_amdgcn_sched_barrier(0);
    logits_mfma_chunk(av1, bv1, acc);
  }

  // Epilogue: lane holds D[p = p0 + 16t + 4g + r][q]; round to fp16, mask the
  // pad columns, store, and keep the first maximum (argmax_key order).
  const bool qok = q < M;
  int best = EXL3_KEY_NONE;
  int besti = 0x7FFFFFFF;
#pragma unroll
  for (int t = 0; t < LG_TILES; ++t) {
    const int64_t pb = p0 + 16 * t + 4 * g;
    uint16_t h[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t p = pb + r;
      const f16 v = (f16)acc[t][r];
      h[r] = (p < n_valid) ? __builtin_bit_cast(uint16_t, v) : (uint16_t)0xFC00;
      if (p < n_pad) argmax_combine(best, besti, argmax_key(h[r]), (int)p);
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
    const int v2 = __shfl_xor(best, o);
    const int i2 = __shfl_xor(besti, o);
    argmax_combine(best, besti, v2, i2);
  }
  if (g == 0 && qok) {  // pairs stored [q][item]: the final pass reads each row contiguously
    pk[(int64_t)q * n_items + item] = best;
    pi[(int64_t)q * n_items + item] = besti;
  }
}

// argmax[q] over the per-wave (key, first index) pairs; any combination order
// gives the same (largest key, smallest index) pair.
__global__ __launch_bounds__(256) void argmax_final_kernel(const int32_t* __restrict__ pk, const int32_t* __restrict__ pi,
                                                           int64_t n_items, int32_t M, int64_t* __restrict__ out) {
  __shared__ int sv[256];
  __shared__ int si[256];
  const int q = blockIdx.x;
  int best = EXL3_KEY_NONE;
  int besti = 0x7FFFFFFF;
  const int32_t* rv = pk + (int64_t)q * n_items;
  const int32_t* ri = pi + (int64_t)q * n_items;
  for (int64_t it = threadIdx.x; it < n_items; it += 256) argmax_combine(best, besti, rv[it], ri[it]);
  sv[threadIdx.x] = best;
  si[threadIdx.x] = besti;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) {
      int b = sv[threadIdx.x];
      int bi = si[threadIdx.x];
      argmax_combine(b, bi, sv[threadIdx.x + s], si[threadIdx.x + s]);
      sv[threadIdx.x] = b;
      si[threadIdx.x] = bi;
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) out[q] = si[0];
}

int64_t logits_items(int64_t n_pad) { return (n_pad + LG_ROWS - 1) / LG_ROWS; }

// fragment-ordered copy of x: 16-row groups, K fp16 each
size_t logits_xperm_bytes(int64_t M, int32_t K) { return (size_t)((M + 15) / 16) * 16 * K * 2; }

hipError_t launch_logits(const uint16_t* x, int32_t M, int32_t K, const uint16_t* w, int64_t n_valid, int64_t n_pad,
                         uint16_t* logits, int64_t ld, int64_t* argmax, int32_t* pk, int32_t* pi, uint16_t* xp,
                         hipStream_t stream, Marks* marks) {
  const int64_t n_items = logits_items(n_pad);
  const bool vec = (ld % 4) == 0 && ((uintptr_t)logits % 8) == 0;
  const int64_t xchunks = (int64_t)logits_xperm_bytes(M, K) / 16;
  logits_xperm_kernel<<<(unsigned)((xchunks + 255) / 256), 256, 0, stream>>>(x, M, K, xp, xchunks);
  hipError_t e0 = hipGetLastError();
  if (e0 != hipSuccess) return e0;
  const unsigned grid = (unsigned)((n_items + LG_WAVES - 1) / LG_WAVES);
  for (int32_t m0 = 0; m0 < M; m0 += 16) {
    hipError_t e = mark_begin(marks, kMarkLogits, stream);
    if (e != hipSuccess) return e;
    logits_kernel<<<grid, 64 * LG_WAVES, 0, stream>>>(xp, M, K, w, n_valid, n_pad, logits, ld, vec, pk, pi, n_items,
                                                      m0);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = mark_end(marks, kMarkLogits, stream);
    if (e != hipSuccess) return e;
  }
  argmax_final_kernel<<<M, 256, 0, stream>>>(pk, pi, n_items, M, argmax);
  return hipGetLastError();
}

// The second argmax stage on its own, for callers with their own first stage
// (the quantized head's pad mask pass).
hipError_t launch_argmax_final(const int32_t* pk, const int32_t* pi, int64_t n_items, int64_t M, int64_t* out,
                               hipStream_t stream) {
  argmax_final_kernel<<<(unsigned)M, 256, 0, stream>>>(pk, pi, n_items, (int32_t)M, out);
  return hipGetLastError();
}

}  // namespace exl3
