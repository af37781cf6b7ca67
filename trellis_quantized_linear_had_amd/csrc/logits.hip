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
// leaves the dot products unchanged). The weights reach the MFMAs through a
// two-slot LDS ring per wave: whole-line non-temporal direct-to-LDS loads fill
// one slot while the MFMAs read their fragments from the other. A pre-pass
// stores x in fragment order (rows past M zero), so each B-fragment load reads
// 1 KiB of contiguous memory instead of 16 rows 2K bytes apart, which measured
// ~40 us slower per call at M = 16 (the row-strided lines crowd a few L2
// channels).
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

// Chunk c of a wave (LG_KC k of its LG_ROWS weight rows, then the chunk's
// LG_STEPS x fragments) goes from global memory straight into the wave's ring
// slot c % 2 by direct-to-LDS loads. Each weight load instruction reads whole
// 128-byte lines, 8 rows x 128 bytes (lane l: row 8 i + l / 8, 16-byte piece
// l % 8), non-temporal: the weights are read once, and a stream of whole
// lines without cache allocation measured 7.0 TB/s against 6.2 with ordinary
// loads (half lines, which the MFMA register layout would need, lose the
// other half without the cache). The piece a lane fetches is XOR-swizzled by
// its row, (row >> 1) & 7, so the fragment reads below (16 consecutive rows,
// one piece) fall on 16 distinct bank groups.
typedef __attribute__((address_space(3))) void lg_lds_void;
#define LG_SLOT_BYTES (LG_ROWS * LG_KC * 2 + LG_STEPS * 1024)  // weights, then x fragments
#define LG_LOADS (LG_ROWS / 8 + LG_STEPS)                      // load instructions per chunk

__device__ __forceinline__ void lg_load_lds16(__amdgpu_buffer_rsrc_t rs, lg_lds_void* dst, uint32_t voff, uint32_t soff,
                                              bool nt) {
  if (nt)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, voff, soff, 0, 2);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, voff, soff, 0, 0);
}

__device__ __forceinline__ int lg_swz(int row) { return (row >> 1) & 7; }

__global__ __launch_bounds__(64 * LG_WAVES) void logits_kernel(const uint16_t* __restrict__ xp, int32_t M, int32_t K,
                                                               const uint16_t* __restrict__ w, int64_t n_valid,
                                                               int64_t n_pad, uint16_t* __restrict__ logits,
                                                               int64_t ld, bool vec_store, int32_t* __restrict__ pk,
                                                               int32_t* __restrict__ pi, int64_t n_items, int32_t m0) {
  __shared__ __attribute__((aligned(16))) char ring[LG_WAVES][2][LG_SLOT_BYTES];
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: scalar resources below
  const int64_t item = (int64_t)blockIdx.x * LG_WAVES + wv;
  if (item >= n_items) return;  // whole wave; no workgroup barriers below
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, pl = lane & 15;
  const int64_t p0 = item * LG_ROWS;
  const int q = m0 + pl;

  f32x4 acc[LG_TILES];
#pragma unroll
  for (int t = 0; t < LG_TILES; ++t) acc[t] = (f32x4){0.f, 0.f, 0.f, 0.f};

  // The wave's rows as one buffer (at most LG_ROWS x K x 2 bytes, below 4 GiB
  // for the entry point's K <= 2^23); rows past
  // the padded width read the wave's first row instead (never stored or
  // ranked), so every load stays inside it.
  const int64_t rows_here = n_pad - p0 < LG_ROWS ? n_pad - p0 : LG_ROWS;
  const __amdgpu_buffer_rsrc_t wrs = make_rsrc(w + p0 * (int64_t)K, (uint32_t)(rows_here * K * 2));
  uint32_t voff[LG_ROWS / 8];  // bytes: row 8 i + lane / 8, piece (lane % 8) ^ swz
#pragma unroll
  for (int i = 0; i < LG_ROWS / 8; ++i) {
    const int r = 8 * i + (lane >> 3);
    voff[i] = (uint32_t)(r < rows_here ? r : 0) * (uint32_t)K * 2u + 16u * (uint32_t)((lane & 7) ^ lg_swz(r));
  }
  // this row group's fragments, K / 32 KiB
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(xp + (int64_t)(m0 / 16) * 16 * K, (uint32_t)(K / 32) * 1024u);
  char* my = ring[wv][0];
  auto issue = [&](int c) {  // chunk c into slot c % 2
    char* slot = my + (c & 1) * LG_SLOT_BYTES;
    const uint32_t kb = (uint32_t)c * LG_KC * 2;  // the chunk's byte offset in a row
#pragma unroll
    for (int i = 0; i < LG_ROWS / 8; ++i) lg_load_lds16(wrs, (lg_lds_void*)(slot + i * 1024), voff[i], kb, true);
#pragma unroll
    for (int st = 0; st < LG_STEPS; ++st)
      lg_load_lds16(xrs, (lg_lds_void*)(slot + LG_ROWS * LG_KC * 2 + st * 1024), (uint32_t)lane * 16,
                    (uint32_t)(c * LG_STEPS + st) * 1024u, false);
  };
  // fragment reads: tile t, step s: row 16 t + pl, piece 4 s + g
  uint32_t aoff[LG_TILES][LG_STEPS];
#pragma unroll
  for (int t = 0; t < LG_TILES; ++t)
#pragma unroll
    for (int st = 0; st < LG_STEPS; ++st) {
      const int r = 16 * t + pl;
      aoff[t][st] = (uint32_t)(r * LG_KC * 2 + 16 * ((4 * st + g) ^ lg_swz(r)));
    }

  const int nc = K / LG_KC;
  issue(0);
  if (nc > 1) issue(1);
  for (int c = 0; c < nc; ++c) {
    // chunk c has landed: only chunk c + 1's loads (issued after it) may be
    // outstanding; on the last chunk none
    if (c + 1 < nc)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LG_LOADS) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    const char* slot = my + (c & 1) * LG_SLOT_BYTES;
    u32x4 bv[LG_STEPS];
#pragma unroll
    for (int st = 0; st < LG_STEPS; ++st)
      bv[st] = *reinterpret_cast<const u32x4*>(slot + LG_ROWS * LG_KC * 2 + st * 1024 + lane * 16);
#pragma unroll
    for (int st = 0; st < LG_STEPS; ++st)
#pragma unroll
      for (int t = 0; t < LG_TILES; ++t) {
        const u32x4 av = *reinterpret_cast<const u32x4*>(slot + aoff[t][st]);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, av), __builtin_bit_cast(f16x8, bv[st]),
                                                        acc[t], 0, 0, 0);
      }
    // every read of the slot has returned (the MFMAs above consumed them)
    // before chunk c + 2's loads overwrite it
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (c + 2 < nc) issue(c + 2);
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
