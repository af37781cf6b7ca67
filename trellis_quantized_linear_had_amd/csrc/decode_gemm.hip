// Fused trellis decode-GEMM for decode-shaped calls (vLLM PR #316, summary and
// "Problem"): each trellis tile is decoded again for every tile of output rows,
// so this path pays more decode work as M rises and serves the calls below the
// row threshold.
//
// Yr = Xr . W with W decoded on the fly. One workgroup per CU (the 128 KiB
// codebook fills most of the 160 KiB LDS); the K x N weight grid is cut into
// ks_count x ns_count rectangles, one per workgroup, so every workgroup decodes
// the same number of tiles. Inside a workgroup the 16 waves form a wn x wk grid
// over (n-tiles, k-steps). Each lane decodes 8 consecutive k of one column and
// feeds them straight into v_mfma_f32_16x16x32_f16 as the B operand (the rows
// of Xr are the A operand, padded to 16). Waves that share n-tiles are summed
// in LDS in a fixed order; each workgroup writes one fp32 partial per output,
// and the finalize kernel sums the ks_count partials in order, applies the
// column scale and the output rotation. No float atomics: bit-identical
// results run to run.
//
// The bound is the codebook gather rate of the LDS (one random 16-bit read
// per weight), not HBM: the packed codes are 0.5 byte per weight.
#include "common.h"
#include "decode_plan.h"
#include "trellis.h"

namespace exl3 {

#define DEC_THREADS 1024
#define DEC_WAVES 16

// Code words per tile and lane: a lane's 8 windows (steps 16c + 8h .. + 7)
// span BITS * 7 + 16 bits from bit BITS (16c + 8h) of the tile; at 4 bits
// that is words d = 2c + h and d + 1 (mod 32), and the lane loads only word
// d: word d + 1 is the one another lane loaded (next_tile_word).
template <int BITS>
struct DecWidth {
  static constexpr int kWords = BITS == 4 ? 1 : TrellisWidth<BITS>::words(8, 8);
};

// An ordinary 32-bit buffer load with cache policy bit 1 set: non-temporal.
__device__ __forceinline__ uint32_t buffer_load_u32_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff_bytes,
                                                       uint32_t soff_bytes) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff_bytes, soff_bytes, 2);
}

// Loads the code words of NT tiles of one k-step, NW per lane. The tile
// bases are wave-uniform (scalar registers); each lane adds a 32-bit offset
// (its k-tile row and word). With 8 or more tiles per wave the loads are
// non-temporal (whole lines read once: 0.6-0.9 us faster per call at 4 bits,
// M = 1..8); the 6-tile instance keeps ordinary loads, which measured faster
// there (a wave past its range re-reads its last tile, which only an
// allocated line serves from the cache).
template <int NT, int NW, int BITS>
__device__ __forceinline__ void decode_load_codes(__amdgpu_buffer_rsrc_t codes, int ntiles_total, int step,
                                                  const int (&tbase)[NT], const int (&loff)[NW],
                                                  uint32_t (&w)[NT][NW]) {
  const uint32_t row = (uint32_t)(2 * step) * ntiles_total * (uint32_t)TrellisWidth<BITS>::kTileBytes;  // bytes
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int j = 0; j < NW; ++j)
      w[t][j] = NT >= 8 ? buffer_load_u32_nt(codes, loff[j], row + tbase[t]) : buffer_load_u32(codes, loff[j], row + tbase[t]);
}

// The A fragments of one k-step (8 consecutive k of one row of Xr, for each
// of the G row groups of the pass) and the step's code words. The A fragments
// go first: loads of one kind retire in order, so the MFMAs of the previous
// step (which need only that step's A fragments) never wait for this step's
// code words. XL (one group): the fragment comes from the workgroup's rotated
// slice in LDS (16-byte chunk j of row m stored at chunk j ^ (m & 15), so the
// 16 rows one read instruction touches fall on distinct banks); otherwise
// from Xr in global memory.
template <int NT, bool XL, int G, int NW, int BITS>
__device__ __forceinline__ void decode_load_step(__amdgpu_buffer_rsrc_t codes, int ntiles_total, int step,
                                                 const int (&tbase)[NT], const int (&loff)[NW],
                                                 const uint16_t* const (&xsrc)[G], int xstep0, const bool (&mok)[G],
                                                 uint32_t (&w)[NT][NW], f16x8 (&a)[G]) {
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if (XL) {
      const int j = 4 * (step - xstep0) + (threadIdx.x & 63) / 16;  // chunk in the row
      a[g] = mok[g] ? *reinterpret_cast<const f16x8*>(xsrc[g] + 8 * (j ^ (threadIdx.x & 15)))
                    : (f16x8){0, 0, 0, 0, 0, 0, 0, 0};
    } else {
      a[g] = mok[g] ? *reinterpret_cast<const f16x8*>(xsrc[g] + 32 * step) : (f16x8){0, 0, 0, 0, 0, 0, 0, 0};
    }
  }
  decode_load_codes<NT, NW, BITS>(codes, ntiles_total, step, tbase, loff, w);
}

// Issues the 8 codebook gathers of one tile; the halves stay unpacked until
// the MFMA that consumes them, so the wait for them can sit right before it.
template <int NW, int BITS>
__device__ __forceinline__ void gather_tile(const uint16_t* cb_lds, const uint32_t (&w)[NW], uint32_t woff,
                                            uint32_t (&g)[8]) {
  uint32_t off[8];
  if constexpr (BITS == 4)
    window_offsets8(w[0], next_tile_word(w[0]), off);  // word d + 1 from its lane
  else
    window_offsets_any<BITS, 8, NW>(w, woff, off);
#pragma unroll
  for (int j = 0; j < 8; ++j) g[j] = lds_cb(cb_lds, off[j]);
}

__device__ __forceinline__ f16x8 pack_tile(const uint32_t (&g)[8]) {
  u32x4 p;
#pragma unroll
  for (int j = 0; j < 4; ++j) p[j] = __builtin_amdgcn_perm(g[2 * j + 1], g[2 * j], 0x05040100u);
  return __builtin_bit_cast(f16x8, p);
}

// The gathers of tile t + 1 are issued before the MFMAs of tile t consume
// tile t, so two tiles' gathers (up to the 15 outstanding LDS reads a wave can
// track) are in flight per wave. Each decoded tile feeds the MFMAs of all G
// row groups: the gathers, the bound, are shared by up to 64 rows.
template <int NT, int G, int NW, int BITS>
__device__ __forceinline__ void decode_mfma_step(const uint16_t* cb_lds, const uint32_t (&w)[NT][NW], uint32_t woff,
                                                 const f16x8 (&a)[G], f32x4 (&acc)[G][NT]) {
  uint32_t cur[8], nxt[8];
  gather_tile<NW, BITS>(cb_lds, w[0], woff, cur);
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (t + 1 < NT) gather_tile<NW, BITS>(cb_lds, w[t + 1], woff, nxt);
    const f16x8 b = pack_tile(cur);
#pragma unroll
    for (int g = 0; g < G; ++g) acc[g][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[g], b, acc[g][t], 0, 0, 0);
    if (t + 1 < NT)
#pragma unroll
      for (int j = 0; j < 8; ++j) cur[j] = nxt[j];
  }
}

template <int NT, bool XL, int G, int BITS>
__global__ __launch_bounds__(DEC_THREADS) void decode_gemm_kernel(const uint16_t* __restrict__ xin,
                                                                  const uint16_t* __restrict__ sign_k,
                                                                  const uint32_t* __restrict__ codes,
                                                                  const uint16_t* __restrict__ cb,
                                                                  float* __restrict__ partials, int32_t K,
                                                                  int32_t N, int32_t ldt, int32_t M,
                                                                  DecodePlan plan) {
  // One 160 KiB block: the codebook (128 KiB), then either the rotated x
  // slice (XL) or the reduction buffer of the multi-group path. After the
  // last gather the whole block serves as reduction slots.
  __shared__ __align__(16) float lds[40960];
  uint16_t* cb_lds = reinterpret_cast<uint16_t*>(lds);
  uint16_t* xs = reinterpret_cast<uint16_t*>(lds + 32768);
  float* red = lds + 32768;

  // N columns are computed (n-tiles 0 .. N/16 - 1); the codes hold ldt
  // n-tiles per k-tile row (ldt >= N / 16: a leading column range of a wider
  // layer)
  const int ksteps_total = K / 32, ntiles_total = ldt;
  const int ks = blockIdx.x / plan.ns_count, ns = blockIdx.x % plan.ns_count;
  const int s_begin = ks * plan.ksteps_per_wg;
  const int s_end = min(s_begin + plan.ksteps_per_wg, ksteps_total);
  const int t_begin = ns * plan.ntiles_per_wg;
  const int t_end = min(t_begin + plan.ntiles_per_wg, N / 16);
  if (s_begin >= s_end || t_begin >= t_end) return;  // whole workgroup idle (uniform)

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int wn_idx = wave % plan.wn, wk_idx = wave / plan.wn;
  const int tw = t_end - t_begin;
  const int per_n = (tw + plan.wn - 1) / plan.wn;
  const int wt_begin = t_begin + min(wn_idx * per_n, tw);
  const int nt_w = min(wt_begin + per_n, t_end) - wt_begin;  // <= NT
  const int sw = s_end - s_begin;
  const int per_k = (sw + plan.wk - 1) / plan.wk;
  const int ws_begin = s_begin + min(wk_idx * per_k, sw);
  const int ws_end = min(ws_begin + per_k, s_end);
  const bool busy = nt_w > 0 && ws_begin < ws_end;  // wave-uniform

  // Lane roles in the 16x16x32 MFMA: A row (= x row) and B column (= n) are
  // lane & 15; the 8-element k slice is lane >> 4: k-tile (lane >> 5) of the
  // step, half (lane >> 4) & 1 of that tile's 16 rows.
  constexpr int NW = DecWidth<BITS>::kWords, TW = TrellisWidth<BITS>::kTileWords;
  const int c = lane & 15;
  const int ktile_in_step = lane >> 5;
  const int wstart = BITS * (16 * c + 8 * ((lane >> 4) & 1));  // first bit of the lane's windows
  const uint32_t woff = (uint32_t)(wstart & 31);
  int loff[NW];  // bytes
#pragma unroll
  for (int j = 0; j < NW; ++j) loff[j] = (ktile_in_step * ntiles_total * TW + (wstart / 32 + j) % TW) * 4;
  const __amdgpu_buffer_rsrc_t crs = make_rsrc(codes, (uint32_t)((int64_t)K * ldt * 16 * BITS / 8));
  // Tiles past the wave's range re-read its last tile (no branches in the
  // hot loop); their sums are never stored.
  int tbase[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) tbase[t] = (wt_begin + min(t, max(nt_w, 1) - 1)) * TrellisWidth<BITS>::kTileBytes;

  // Prologue. The codebook copy is in flight while (XL) the workgroup
  // rotates its x slice: rows < M, k in [32 s_begin, 32 s_end), 16 lanes per
  // 128-element block, the same arithmetic as the stand-alone rotation pass
  // (sign bit flip, fp32 butterflies, one scaling, one fp16 rounding).
  {
    const u32x4* src = reinterpret_cast<const u32x4*>(cb);
    u32x4* dst = reinterpret_cast<u32x4*>(cb_lds);
    constexpr int kPer = 65536 * 2 / 16 / DEC_THREADS;
    u32x4 tmp[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) tmp[i] = src[threadIdx.x + i * DEC_THREADS];
    if (XL) {
      // M * kslice <= DEC_XS_BYTES / 2 elements, so each 16-lane group has
      // at most two (row, block) tasks; both loads go out before any math.
      static_assert(DEC_XS_BYTES / 2 / 128 <= 2 * (DEC_THREADS / 16), "more than two rotation tasks per group");
      const int kslice = sw * 32, nblk = sw / 4, ntask = M * nblk;
      const int q = threadIdx.x & 15;
      // Without signs the mask is zero (the second load then re-reads x).
      const uint16_t* sgn = sign_k ? sign_k : xin;
      const uint32_t smask = sign_k ? 0x80008000u : 0u;
      u32x4 xv[2], sv[2];
      int xoff[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int task = (threadIdx.x >> 4) + i * (DEC_THREADS / 16);
        const int tk = task < ntask ? task : 0;
        const int m = tk / nblk, b = tk - m * nblk;
        const int64_t kg = (int64_t)s_begin * 32 + 128 * b + 8 * q;
        xv[i] = *reinterpret_cast<const u32x4*>(xin + (int64_t)m * K + kg);
        sv[i] = *reinterpret_cast<const u32x4*>(sgn + kg);
        xoff[i] = task < ntask ? m * kslice + 8 * (16 * b + (q ^ (m & 15))) : -1;
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if (xoff[i] >= 0) {  // uniform over the 16 lanes of the block
          xv[i] ^= sv[i] & smask;  // +-1: flip the sign bit
          float v[8];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            v[2 * j] = bits_lo_f16(xv[i][j]);
            v[2 * j + 1] = bits_hi_f16(xv[i][j]);
          }
          wht128_16(v, q);
          u32x4 o;
#pragma unroll
          for (int j = 0; j < 4; ++j)
            o[j] = pack_f16x2(v[2 * j] * EXL3_INV_SQRT128, v[2 * j + 1] * EXL3_INV_SQRT128);
          *reinterpret_cast<u32x4*>(xs + xoff[i]) = o;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) dst[threadIdx.x + i * DEC_THREADS] = tmp[i];
  }
  // (The first step's code words are not requested before this barrier: its
  // release fence would wait for them.)
  __syncthreads();

  // Fixed-order reduction over the wk waves that share these n-tiles, for
  // the 16 rows m0g .. m0g + 15: sum = ((w_0 + w_1) + w_2) + ... over the
  // waves' k order, for every output. D layout of the MFMA: lane holds rows
  // 4*(lane>>4) + r, column lane & 15. `dead`: no gather follows, so the whole
  // LDS block holds one slot per (wave, tile) and all waves store at once, in
  // passes of `chunk` tiles; otherwise (the codebook is still needed) the
  // slots go to the 32 KiB beside the codebook: all at once when the wk slots
  // of every tile fit there, else the waves accumulate one at a time.
  const int eoff = 4 * (lane >> 4) * 16 + c;
  const int wt_off = wt_begin - t_begin;
  auto reduce_store = [&](const f32x4 (&accg)[NT], int m0g, bool dead) {
    if (dead) {
      float* slots = lds;
      const int chunk = 40960 / 256 / plan.wk;
      __syncthreads();
      for (int t0 = 0; t0 < tw; t0 += chunk) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const int tt = wt_off + t - t0;
          if (t < nt_w && tt >= 0 && tt < chunk)
#pragma unroll
            for (int r = 0; r < 4; ++r) slots[(wk_idx * chunk + tt) * 256 + eoff + r * 16] = accg[t][r];
        }
        __syncthreads();
        const int nout = min(chunk, tw - t0) * 256;
        for (int idx = threadIdx.x; idx < nout; idx += DEC_THREADS) {
          float sum = slots[idx];
          for (int j = 1; j < plan.wk; ++j) sum += slots[j * chunk * 256 + idx];
          const int t = t0 + (idx >> 8), e = idx & 255, m = m0g + (e >> 4), n = (t_begin + t) * 16 + (e & 15);
          if (m < M) partials[((int64_t)ks * M + m) * N + n] = sum;
        }
        __syncthreads();
      }
    } else if (plan.wk * tw * 256 <= 8192) {
      // The wk slots of every tile fit beside the codebook: all waves store
      // at once and every thread sums the slots in wave order (the same sums
      // as the one-wave-at-a-time loop below, without its wk barriers).
#pragma unroll
      for (int t = 0; t < NT; ++t)
        if (t < nt_w)
#pragma unroll
          for (int r = 0; r < 4; ++r) red[(wk_idx * tw + wt_off + t) * 256 + eoff + r * 16] = accg[t][r];
      __syncthreads();
      for (int idx = threadIdx.x; idx < tw * 256; idx += DEC_THREADS) {
        float sum = red[idx];
        for (int j = 1; j < plan.wk; ++j) sum += red[j * tw * 256 + idx];
        const int t = idx >> 8, e = idx & 255, m = m0g + (e >> 4), n = (t_begin + t) * 16 + (e & 15);
        if (m < M) partials[((int64_t)ks * M + m) * N + n] = sum;
      }
      __syncthreads();
    } else {
      const int rbase = wt_off * 256 + eoff;
      for (int j = 0; j < plan.wk; ++j) {
        if (wk_idx == j) {
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            if (t < nt_w) {
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                float* p = &red[rbase + t * 256 + r * 16];
                *p = (j == 0) ? accg[t][r] : *p + accg[t][r];
              }
            }
          }
        }
        __syncthreads();
      }
      // partials[ks][m][n]
      for (int idx = threadIdx.x; idx < tw * 256; idx += DEC_THREADS) {
        const int t = idx >> 8, e = idx & 255, m = m0g + (e >> 4), n = (t_begin + t) * 16 + (e & 15);
        if (m < M) partials[((int64_t)ks * M + m) * N + n] = red[idx];
      }
      __syncthreads();
    }
  };

  // Passes of G row groups (16 rows each) over the wave's tiles and k range.
  for (int m0 = 0; m0 < M; m0 += 16 * G) {
    f32x4 acc[G][NT];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[g][t] = (f32x4){0.f, 0.f, 0.f, 0.f};

    // XL: the row of the LDS slice; otherwise the row of Xr in global memory
    // at this lane's 8-element k offset.
    bool mok[G];
    const uint16_t* xsrc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int mrow = m0 + 16 * g + c;
      mok[g] = mrow < M;
      xsrc[g] = XL ? xs + (mok[g] ? mrow : 0) * (sw * 32) : xin + (int64_t)(mok[g] ? mrow : 0) * K + 8 * (lane >> 4);
    }
    if (busy) {
      uint32_t w0[NT][NW], w1[NT][NW];
      f16x8 a0[G], a1[G];
      const int last = ws_end - 1;
      decode_load_step<NT, XL, G, NW, BITS>(crs, ntiles_total, ws_begin, tbase, loff, xsrc, s_begin, mok, w0, a0);
      // Pairs of k steps with no branch inside: each step's code words are
      // requested before the previous step decodes. (With the second half of
      // a pair under a branch, the compiler sank the loads of w1 into it, past
      // the decode of w0, so every other step waited a full memory round trip
      // for its words.) An odd step count ends with one step whose words are
      // already in w0.
      int step = ws_begin;
      for (; step + 1 < ws_end; step += 2) {
        decode_load_step<NT, XL, G, NW, BITS>(crs, ntiles_total, step + 1, tbase, loff, xsrc, s_begin, mok, w1, a1);
        decode_mfma_step<NT, G, NW, BITS>(cb_lds, w0, woff, a0, acc);
        decode_load_step<NT, XL, G, NW, BITS>(crs, ntiles_total, min(step + 2, last), tbase, loff, xsrc, s_begin,
                                              mok, w0, a0);
        decode_mfma_step<NT, G, NW, BITS>(cb_lds, w1, woff, a1, acc);
      }
      if (step < ws_end) decode_mfma_step<NT, G, NW, BITS>(cb_lds, w0, woff, a0, acc);
    }

    const bool dead = m0 + 16 * G >= M;  // last pass: the codebook is no longer read
#pragma unroll
    for (int g = 0; g < G; ++g)
      if (m0 + 16 * g < M) reduce_store(acc[g], m0 + 16 * g, dead);  // uniform
  }
}

// Output stage: y[m][128b + i] = fp16(s_N * (1/sqrt128) * sum_j H[i][j] *
// scale[n_j] * sum_ks partials[ks][m][n_j]); 16 lanes per (row, 128-column
// block), 8 columns per lane. The partials are summed in ks order; the loads
// of the column scales and signs and of up to 8 slices are all issued before
// any of them is used, so one memory round trip serves them.
__global__ __launch_bounds__(256) void decode_finalize_kernel(const float* __restrict__ partials, int32_t ks_count,
                                                              const uint16_t* __restrict__ scale,
                                                              const uint16_t* __restrict__ sign_n,
                                                              uint16_t* __restrict__ y, int64_t ldy, int32_t M,
                                                              int32_t N) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int q = (int)(gid & 15);
  const int64_t nblocks = (int64_t)M * (N / 128);
  const int64_t blk_raw = gid >> 4;
  const int64_t blk = blk_raw < nblocks ? blk_raw : nblocks - 1;
  const int64_t m = blk / (N / 128);
  const int64_t n0 = (blk % (N / 128)) * 128 + 8 * q;
  const int64_t slice = (int64_t)M * N;
  const u32x4 sc = *reinterpret_cast<const u32x4*>(scale + n0);
  // without signs the scales are read again and masked to zero (no branch
  // between the loads and their use)
  const u32x4 sg = *reinterpret_cast<const u32x4*>((sign_n ? sign_n : scale) + n0);
  const uint32_t smask = sign_n ? 0x80008000u : 0u;

  float v[8];
  const f32x4* src = reinterpret_cast<const f32x4*>(partials + m * N + n0);
  // slices 0 .. 7 in one batch (slice 0 assigned, the rest added in order),
  // then further batches of 8
  auto batch = [&](int k0) {
    f32x4 p[8][2];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int k = min(k0 + i, ks_count - 1);
      p[i][0] = src[k * slice / 4];
      p[i][1] = src[k * slice / 4 + 1];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (k0 + i == 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[j] = p[i][0][j];
          v[4 + j] = p[i][1][j];
        }
      } else if (k0 + i < ks_count) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[j] += p[i][0][j];
          v[4 + j] += p[i][1][j];
        }
      }
    }
  };
  batch(0);
  for (int k0 = 8; k0 < ks_count; k0 += 8) batch(k0);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[2 * j] *= bits_lo_f16(sc[j]);
    v[2 * j + 1] *= bits_hi_f16(sc[j]);
  }
  wht128_16(v, q);
  u32x4 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) o[j] = pack_f16x2(v[2 * j] * EXL3_INV_SQRT128, v[2 * j + 1] * EXL3_INV_SQRT128);
  o ^= sg & smask;
  if (blk_raw < nblocks) *reinterpret_cast<u32x4*>(y + m * ldy + n0) = o;
}

hipError_t launch_decode_gemm(const uint16_t* xin, const uint16_t* sign_k, const uint32_t* codes, const uint16_t* cb,
                              float* partials, int32_t K, int32_t N, int32_t ldt, int32_t M, int32_t bits,
                              const DecodePlan& plan, hipStream_t stream) {
  const int grid = plan.ks_count * plan.ns_count;
#define EXL3_DEC_LAUNCH(nt, xl, g, b)                                                                          \
  decode_gemm_kernel<nt, xl, g, b><<<grid, DEC_THREADS, 0, stream>>>(xin, sign_k, codes, cb, partials, K, N, ldt, M, \
                                                                     plan)
#define EXL3_DEC_CASE1(nt, b)          \
  case nt:                             \
    if (plan.x_in_lds)                 \
      EXL3_DEC_LAUNCH(nt, true, 1, b); \
    else                               \
      EXL3_DEC_LAUNCH(nt, false, 1, b);\
    break;
#define EXL3_DEC_CASEG(nt, g)         \
  case nt:                            \
    EXL3_DEC_LAUNCH(nt, false, g, 4); \
    break;
#define EXL3_DEC_CASEGB(nt, g, b)      \
  case nt:                             \
    EXL3_DEC_LAUNCH(nt, false, g, b);  \
    break;
#define EXL3_DEC_OTHER(b)                                               \
  case b:                                                               \
    if (plan.groups == 1) {                                             \
      switch (plan.nt_wave) {                                           \
        EXL3_DEC_CASE1(2, b)                                            \
        EXL3_DEC_CASE1(3, b)                                            \
        EXL3_DEC_CASE1(4, b)                                            \
        EXL3_DEC_CASE1(5, b)                                            \
        EXL3_DEC_CASE1(6, b)                                            \
        default:                                                        \
          return hipErrorInvalidValue;                                  \
      }                                                                 \
    } else if (plan.groups == 2 && !plan.x_in_lds) {                    \
      switch (plan.nt_wave) {                                           \
        EXL3_DEC_CASEGB(2, 2, b)                                        \
        EXL3_DEC_CASEGB(3, 2, b)                                        \
        EXL3_DEC_CASEGB(4, 2, b)                                        \
        EXL3_DEC_CASEGB(5, 2, b)                                        \
        default:                                                        \
          return hipErrorInvalidValue;                                  \
      }                                                                 \
    } else if (plan.groups == 4 && !plan.x_in_lds) {                    \
      switch (plan.nt_wave) {                                           \
        EXL3_DEC_CASEGB(1, 4, b)                                        \
        EXL3_DEC_CASEGB(2, 4, b)                                        \
        default:                                                        \
          return hipErrorInvalidValue;                                  \
      }                                                                 \
    } else {                                                            \
      return hipErrorInvalidValue;                                      \
    }                                                                   \
    break;
  if (bits != 4) {
    switch (bits) {
      EXL3_DEC_OTHER(1)
      EXL3_DEC_OTHER(2)
      EXL3_DEC_OTHER(3)
      EXL3_DEC_OTHER(5)
      EXL3_DEC_OTHER(6)
      EXL3_DEC_OTHER(7)
      EXL3_DEC_OTHER(8)
      default:
        return hipErrorInvalidValue;
    }
  } else if (plan.groups == 1) {
    switch (plan.nt_wave) {
      EXL3_DEC_CASE1(1, 4)
      EXL3_DEC_CASE1(2, 4)
      EXL3_DEC_CASE1(3, 4)
      EXL3_DEC_CASE1(4, 4)
      EXL3_DEC_CASE1(5, 4)
      EXL3_DEC_CASE1(6, 4)
      EXL3_DEC_CASE1(8, 4)
      EXL3_DEC_CASE1(9, 4)
      EXL3_DEC_CASE1(10, 4)
      default:
        return hipErrorInvalidValue;
    }
  } else if (plan.groups == 2 && !plan.x_in_lds) {
    switch (plan.nt_wave) {
      EXL3_DEC_CASEG(1, 2)
      EXL3_DEC_CASEG(2, 2)
      EXL3_DEC_CASEG(3, 2)
      EXL3_DEC_CASEG(4, 2)
      EXL3_DEC_CASEG(5, 2)
      default:
        return hipErrorInvalidValue;
    }
  } else if (plan.groups == 4 && !plan.x_in_lds) {
    switch (plan.nt_wave) {
      EXL3_DEC_CASEG(1, 4)
      EXL3_DEC_CASEG(2, 4)
      EXL3_DEC_CASEG(3, 4)
      default:
        return hipErrorInvalidValue;
    }
  } else {
    return hipErrorInvalidValue;
  }
#undef EXL3_DEC_OTHER
#undef EXL3_DEC_CASEGB
#undef EXL3_DEC_CASEG
#undef EXL3_DEC_CASE1
#undef EXL3_DEC_LAUNCH
  return hipGetLastError();
}

hipError_t launch_decode_finalize(const float* partials, int32_t ks_count, const uint16_t* scale,
                                  const uint16_t* sign_n, uint16_t* y, int64_t ldy, int32_t M, int32_t N,
                                  hipStream_t stream) {
  const int64_t threads = (int64_t)M * (N / 128) * 16;
  decode_finalize_kernel<<<(unsigned)((threads + 255) / 256), 256, 0, stream>>>(partials, ks_count, scale, sign_n,
                                                                                y, ldy, M, N);
  return hipGetLastError();
}

}  // namespace exl3
