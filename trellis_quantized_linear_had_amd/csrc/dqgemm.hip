// Dequant-in-GEMM: the layer for row counts from a few dozen to thousands,
// with W decoded from the packed trellis codes inside the MFMA loop and never
// written out (vLLM PR #316, follow-up item 4: the Hadamard + reconstruct
// share of the prefill call is the part a fused dequant-GEMM removes;
// "Kernel measurements": the unexported reconstruct_had_slice).
//
// Transposed product, as in the prefill GEMM: D[p][q] = sum_k W[k][p] Xr[q][k]
// with v_mfma_f32_32x32x16_f16, A = 32 columns p x 16 k of W decoded in
// registers, B = 32 rows q x 16 k of Xr in the 32-row fragment order the
// rotation pass writes (1 KiB per fragment, one contiguous load).
//
// The cost is one random 16-bit codebook read from LDS per decoded weight,
// and each decoded A fragment feeds the MFMAs of every row fragment the wave
// holds: a wave owns 64 columns (two A fragments) and up to 256 rows (eight B
// fragments), so a weight is decoded once per 256 rows. The 2 x 8
// accumulator tiles take 256 registers, so there is one wave per SIMD (four
// per workgroup, one workgroup per CU: the 128 KiB codebook fills the LDS).
// A lane of A fragment f holds 8 consecutive k of column p: the windows of
// steps 16 c + 8 h .. + 7 of one 16 x 16 trellis tile, two code words at 4
// bits.
//
// Work: a unit is 256 columns (four waves of 64) by one pass of R = 32 NQB
// rows. The first `full` units (pass-major) each take one workgroup over all
// of K, which applies the column scales, the output rotation (a 128-column
// block spans two waves: they swap halves of their accumulators through the
// LDS the codebook no longer needs) and the signs, and stores fp16 y. The
// remaining `tail` units are split along K into tail_ks pieces, which store
// fp32 partial sums; dq_fixup_kernel adds each unit's pieces in k order and
// runs the same output stage.
#include <type_traits>

#include "common.h"
#include "dq_plan.h"
#include "epilogue.h"
#include "trellis.h"

namespace exl3 {

#define DQ_THREADS 256
#define DQ_COLS_WAVE 64
#define DQ_COLS_WG 256

typedef __attribute__((address_space(3))) void dq_lds_void;

// Code words of one 16-k step for the wave's two A fragments: lane (c, tile
// parity, half h) needs words 2c + h and 2c + h + 1 (mod 32) of its tile.
__device__ __forceinline__ void dq_load_codes(__amdgpu_buffer_rsrc_t rs, uint32_t row_off, const uint32_t (&voff)[2][2],
                                              uint32_t (&w)[2][2]) {
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int j = 0; j < 2; ++j) w[f][j] = buffer_load_u32(rs, voff[f][j], row_off);
}

// The 8 codebook reads of one A fragment.
__device__ __forceinline__ void dq_gather(const uint16_t* cb_lds, const uint32_t (&w)[2], uint32_t (&g)[8]) {
  uint32_t off[8];
  window_offsets8(w[0], w[1], off);
#pragma unroll
  for (int j = 0; j < 8; ++j) g[j] = lds_cb(cb_lds, off[j]);
}

// The 8 reads packed as the MFMA's f16x8.
__device__ __forceinline__ f16x8 dq_pack(const uint32_t (&g)[8]) {
  u32x4 p;
#pragma unroll
  for (int j = 0; j < 4; ++j) p[j] = __builtin_amdgcn_perm(g[2 * j + 1], g[2 * j], 0x05040100u);
  return __builtin_bit_cast(f16x8, p);
}

// t[f] *= the scale of its column: p = p0 + 32 f + 8 (r >> 2) + 4 lhalf + (r & 3).
__device__ __forceinline__ void dq_scale_tiles(f32x16 (&t)[2], const uint16_t* __restrict__ scale, int p0, int lane) {
  const int lhalf = lane >> 5;
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    u32x2 sc[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) sc[g] = *reinterpret_cast<const u32x2*>(scale + p0 + 32 * f + 8 * g + 4 * lhalf);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      t[f][4 * g] *= bits_lo_f16(sc[g][0]);
      t[f][4 * g + 1] *= bits_hi_f16(sc[g][0]);
      t[f][4 * g + 2] *= bits_lo_f16(sc[g][1]);
      t[f][4 * g + 3] *= bits_hi_f16(sc[g][1]);
    }
  }
}

// TAIL = false: workgroup w computes whole unit w; TAIL = true: workgroup w
// computes piece w % tail_ks of tail unit full + w / tail_ks. (One kernel with
// both output stages ran out of registers where the two paths join.)
template <int NQB, bool TAIL>
__global__ __launch_bounds__(DQ_THREADS) __attribute__((amdgpu_waves_per_eu(1, 1))) void dqgemm_kernel(
    const uint16_t* __restrict__ xf, const uint32_t* __restrict__ codes, const uint16_t* __restrict__ cb,
    const uint16_t* __restrict__ scale, const uint16_t* __restrict__ sign_n, uint16_t* __restrict__ y, int64_t ldy,
    float* __restrict__ partials, int32_t K, int32_t N, int32_t ldt, int32_t M, DqPlan plan) {
  // the codebook; after the last read, the accumulator exchange of the output stage
  __shared__ __align__(16) uint16_t cb_lds[65536];

  constexpr int R = 32 * NQB;
  const int ksub = K / 16;
  const int w = blockIdx.x;
  int unit, s_begin, s_end;
  if (!TAIL) {
    unit = w;
    s_begin = 0;
    s_end = ksub;
  } else {
    const int t = w / plan.tail_ks, piece = w % plan.tail_ks;
    unit = plan.full + t;
    s_begin = piece * plan.ksub_per_piece;
    s_end = min(s_begin + plan.ksub_per_piece, ksub);
  }
  const int pass = unit / plan.pblocks, pb = unit % plan.pblocks;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int p0_raw = pb * DQ_COLS_WG + wave * DQ_COLS_WAVE;
  const bool pvalid = p0_raw < N;                      // N is a multiple of 128: valid waves come in pairs
  const int p0 = pvalid ? p0_raw : N - DQ_COLS_WAVE;  // idle waves re-read the last group, never store

  // Codebook into LDS straight from global memory (1 KiB per wave
  // instruction), while the first code words and row fragments are requested.
  {
    const char* src = reinterpret_cast<const char*>(cb) + threadIdx.x * 16;
#pragma unroll 4
    for (int i = 0; i < 65536 * 2 / (DQ_THREADS * 16); ++i)
      __builtin_amdgcn_global_load_lds(src + i * DQ_THREADS * 16,
                                       (dq_lds_void*)(reinterpret_cast<char*>(cb_lds) + i * DQ_THREADS * 16 +
                                                      wave * 1024),
                                       16, 0, 0);
  }

  // Lane roles: A row p = lane % 32 -> n-tile (p0 + 32 f) / 16 + (lane >> 4 & 1),
  // tile column c = lane & 15, k half h = lane >> 5.
  const int c = lane & 15, h = lane >> 5, tpar = (lane >> 4) & 1;
  const int d = 2 * c + h;
  uint32_t voff[2][2];
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    const int nt = (p0 + 32 * f) / 16 + tpar;
    voff[f][0] = (uint32_t)(nt * 128 + 4 * d);
    voff[f][1] = (uint32_t)(nt * 128 + 4 * ((d + 1) & 31));
  }
  const __amdgpu_buffer_rsrc_t crs = make_rsrc(codes, (uint32_t)((int64_t)K * ldt * 8));
  const uint32_t row_bytes = (uint32_t)ldt * 128;  // one k-tile row of codes

  // Row fragments: blocks pass * NQB + j, clamped to the last block of the
  // padded rows (rows past M are zero or repeats and are never stored).
  const int nqb_all = (M + 31) / 32;
  const uint16_t* bsrc[NQB];
#pragma unroll
  for (int j = 0; j < NQB; ++j) {
    const int qb = min(pass * NQB + j, nqb_all - 1);
    bsrc[j] = xf + ((int64_t)qb * ksub * 64 + lane) * 8;
  }
  auto frag = [&](int j, int s) { return *reinterpret_cast<const f16x8*>(bsrc[j] + (int64_t)s * 512); };

  f32x16 acc[2][NQB];
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int j = 0; j < NQB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[f][j][r] = 0.f;

  // Rings: the code words of steps s .. s + 3 (HBM latency is longer than a
  // step) and the row fragments of steps s and s + 1; the loop is unrolled by
  // four so every ring slot is a fixed set of registers.
  uint32_t wr[4][2][2];
  f16x8 br[2][NQB];
#pragma unroll
  for (int u = 0; u < 4; ++u) dq_load_codes(crs, (uint32_t)min(s_begin + u, s_end - 1) * row_bytes, voff, wr[u]);
#pragma unroll
  for (int j = 0; j < NQB; ++j) br[0][j] = frag(j, s_begin);
  __builtin_amdgcn_s_waitcnt(0);  // the codebook's direct-to-LDS loads (and the rest) have landed
  __syncthreads();

  uint32_t g[2][8];
  dq_gather(cb_lds, wr[0][0], g[0]);
  dq_gather(cb_lds, wr[0][1], g[1]);

  // Step s (ring phase U = (s - s_begin) % 4): pack the codebook reads of s,
  // then its 2 x NQB MFMAs, each followed (one wave per SIMD: the matrix unit
  // only works while this wave issues MFMAs) by one small piece of the next
  // step's work, in source order fenced by scheduling barriers: after the
  // even MFMAs a row fragment of s + 1, after the odd ones the window offsets
  // and codebook reads of s + 1 and the code words of s + 4. (Left to itself
  // the compiler moved row-fragment loads next to their MFMAs.)
  auto step = [&](auto U, int s) {
    constexpr int u = decltype(U)::value;
    const int s1 = min(s + 1, s_end - 1), s4 = min(s + 4, s_end - 1);
    const f16x8 a0 = dq_pack(g[0]), a1 = dq_pack(g[1]);
    uint32_t off[2][8];
    auto work = [&](int k) {  // k: the odd MFMA slot, 0 .. NQB - 1
      constexpr int W = NQB;
      // pieces: 0 offsets f0, 1-2 reads f0, 3 offsets f1, 4-5 reads f1, 6 code words
      const int piece_lo = k * 7 / W, piece_hi = (k + 1) * 7 / W;
      for (int pc = piece_lo; pc < piece_hi; ++pc) {
        if (pc == 0) window_offsets8(wr[(u + 1) & 3][0][0], wr[(u + 1) & 3][0][1], off[0]);
        if (pc == 3) window_offsets8(wr[(u + 1) & 3][1][0], wr[(u + 1) & 3][1][1], off[1]);
        if (pc == 1 || pc == 2 || pc == 4 || pc == 5) {
          const int f = pc >= 4, half = (pc - 1) % 3;
#pragma unroll
          for (int i = 0; i < 4; ++i) g[f][4 * half + i] = lds_cb(cb_lds, off[f][4 * half + i]);
        }
        if (pc == 6) dq_load_codes(crs, (uint32_t)s4 * row_bytes, voff, wr[u]);
      }
    };
#pragma unroll
    for (int j = 0; j < NQB; ++j) {
      acc[0][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, br[u & 1][j], acc[0][j], 0, 0, 0);
      br[(u + 1) & 1][j] = frag(j, s1);
      __builtin_amdgcn_sched_barrier(0);
      acc[1][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, br[u & 1][j], acc[1][j], 0, 0, 0);
      work(j);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  using U0 = std::integral_constant<int, 0>;
  using U1 = std::integral_constant<int, 1>;
  using U2 = std::integral_constant<int, 2>;
  using U3 = std::integral_constant<int, 3>;
  // every k range is a whole number of 4-step blocks (K is a multiple of 128
  // and the plan cuts K in multiples of 4 steps)
  for (int s = s_begin; s < s_end; s += 4) {
    step(U0{}, s);
    step(U1{}, s + 1);
    step(U2{}, s + 2);
    step(U3{}, s + 3);
  }

  if (TAIL) {
    // A tail piece: partials[w][q][p] over the unit's R rows and 256
    // columns; lane holds D[p = 8 (r >> 2) + 4 h + (r & 3)][q = lane % 32] of
    // tile (f, j).
    if (!pvalid) return;
    float* base = partials + (int64_t)w * R * DQ_COLS_WG + wave * DQ_COLS_WAVE + 4 * h;
#pragma unroll
    for (int j = 0; j < NQB; ++j) {
      float* dst = base + (32 * j + (lane & 31)) * DQ_COLS_WG;
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const f32x4 v = {acc[f][j][4 * g4], acc[f][j][4 * g4 + 1], acc[f][j][4 * g4 + 2], acc[f][j][4 * g4 + 3]};
          *reinterpret_cast<f32x4*>(dst + 32 * f + 8 * g4) = v;
        }
    }
    return;
  }

  // A whole unit: the output stage here. Waves 2b and 2b + 1 hold the two
  // 64-column halves of rotation block b for all R rows. Butterfly stages on
  // different index bits commute, so each wave scales its tiles and runs the
  // six stages inside its half, and parks them in the LDS the codebook no
  // longer needs; after a barrier, one wave of the pair adds and subtracts
  // the halves (the seventh stage) and stores. Two row fragments per round
  // keep few registers live across the barriers: slots [wave][jj][f][4][64]
  // of f32x4, 64 KiB.
  f32x4* xch = reinterpret_cast<f32x4*>(cb_lds);
  const int odd = wave & 1;
  const int pwb = pb * DQ_COLS_WG + (wave & ~1) * DQ_COLS_WAVE;  // the block's first column
  auto slot_of = [&](int wv, int jj, int f, int v) { return (((wv * 2 + jj) * 2 + f) * 4 + v) * 64 + lane; };
  __syncthreads();  // every wave is done with the codebook
#pragma unroll
  for (int r = 0; r < (NQB + 1) / 2; ++r) {
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int j = 2 * r + jj;
      if (j >= NQB) continue;
      // (fenced: hoisting later rounds' accumulator reads overflows the registers)
      __builtin_amdgcn_sched_barrier(0);
      f32x16 t[2] = {acc[0][j], acc[1][j]};
      dq_scale_tiles(t, scale, p0, lane);
      wht64_half(t, lane);
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          xch[slot_of(wave, jj, f, v)] = (f32x4){t[f][4 * v], t[f][4 * v + 1], t[f][4 * v + 2], t[f][4 * v + 3]};
    }
    __syncthreads();
    const int j = 2 * r + odd;  // the even wave stores fragment 2r, the odd one 2r + 1
    if (pvalid && j < NQB) {
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        f32x16 lo, hi;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const f32x4 a = xch[slot_of(wave & ~1, odd, f, v)], b = xch[slot_of(wave | 1, odd, f, v)];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            lo[4 * v + e] = a[e];
            hi[4 * v + e] = b[e];
          }
        }
        store_halves_tile(lo, hi, f, lane, pwb, pass * R + 32 * j, N, M, y, ldy, 0, sign_n);
      }
    }
    __syncthreads();  // the slots are rewritten in the next round
  }
}

// ---- Eight-wave form: 32 columns per wave (two 16-column A fragments of
// v_mfma_f32_16x16x32_f16), one pass of R = 16 NQ rows (NQ = 4, 8 or 16 row
// fragments), the pass's rows of Xr staged once per workgroup in the LDS
// beside the codebook (16-row fragment order, two stages of 16 fragments:
// one, two or four 32-k steps each), so each wave reads them from LDS
// instead of loading them itself, and two waves per SIMD hide each other's
// waits. A lane of A fragment f holds 8 consecutive k of column p: k-tile
// (lane >> 5) of the step, half (lane >> 4) & 1 of that tile's 16 steps. The
// tail is split into equal pieces per unit or dealt stream-K (DqPlan).
#define DQ2_THREADS 512

// One direct-to-LDS buffer load of 16 bytes per lane (lane i's bytes land at
// dst + 16 i). A plain function: called with arguments that depend on a
// kernel template's parameters, the builtin made the compiler drop that
// template's instantiations without a diagnostic.
__device__ __forceinline__ void dq_buffer_load_lds16(__amdgpu_buffer_rsrc_t rs, dq_lds_void* dst, uint32_t voff,
                                                     uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, voff, soff, 0, 0);
}

template <int NQ, bool TAIL>
__global__ __launch_bounds__(DQ2_THREADS) __attribute__((amdgpu_waves_per_eu(2, 2))) void dqgemm2_kernel(
    const uint16_t* __restrict__ xf, const uint32_t* __restrict__ codes, const uint16_t* __restrict__ cb,
    const uint16_t* __restrict__ scale, const uint16_t* __restrict__ sign_n, uint16_t* __restrict__ y, int64_t ldy,
    float* __restrict__ partials, int32_t K, int32_t N, int32_t ldt, int32_t M, DqPlan plan) {
  static_assert(NQ == 4 || NQ == 8 || NQ == 16, "row fragments per pass");
  constexpr int R = 16 * NQ;     // rows per pass
  constexpr int SPB = 16 / NQ;   // 32-k steps per x stage: every stage holds 16 fragments (16 KiB)
  constexpr int XSTAGE = 16 * 512;  // halves per x stage
  // the codebook, then two x stages; after the last codebook read, the output stage's transpose buffer
  __shared__ __align__(16) uint16_t lds[65536 + 2 * XSTAGE];
  uint16_t* cb_lds = lds;
  uint16_t* xs = lds + 65536;

  const int ks32 = K / 32;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // Codebook into LDS straight from global memory (1 KiB per wave instruction).
  {
    const char* src = reinterpret_cast<const char*>(cb) + threadIdx.x * 16;
#pragma unroll 4
    for (int i = 0; i < 65536 * 2 / (DQ2_THREADS * 16); ++i)
      __builtin_amdgcn_global_load_lds(
          src + i * DQ2_THREADS * 16,
          (dq_lds_void*)(reinterpret_cast<char*>(cb_lds) + i * DQ2_THREADS * 16 + wave * 1024), 16, 0, 0);
  }

  // This workgroup's work: one segment (a unit and a range of its 32-k steps),
  // or two when a stream-K run crosses from one tail unit into the next.
  int unit0, b0, e0, unit1 = 0, e1 = 0, nseg = 1;
  if (!TAIL) {
    unit0 = blockIdx.x;
    b0 = 0;
    e0 = ks32;
  } else if (plan.sk_steps == 0) {
    const int t = blockIdx.x / plan.tail_ks, piece = blockIdx.x % plan.tail_ks;
    unit0 = plan.full + t;
    b0 = piece * (plan.ksub_per_piece / 2);  // ksub_per_piece: 16-k steps, whole x stages
    e0 = min(b0 + plan.ksub_per_piece / 2, ks32);
  } else {
    // steps [g0, g1) of the tail units' 32-k steps, unit-major
    const int64_t total = (int64_t)plan.tail * ks32;
    const int64_t g0 = (int64_t)blockIdx.x * plan.sk_steps, g1 = min(g0 + plan.sk_steps, total);
    const int t0 = (int)(g0 / ks32);
    unit0 = plan.full + t0;
    b0 = (int)(g0 - (int64_t)t0 * ks32);
    e0 = (int)min((int64_t)ks32, b0 + (g1 - g0));
    if (g0 + (e0 - b0) < g1) {  // sk_steps <= K / 32: the run ends in the next unit
      unit1 = unit0 + 1;
      e1 = (int)(g1 - g0 - (e0 - b0));
      nseg = 2;
    }
  }

  for (int seg = 0; seg < nseg; ++seg) {  // uniform
    const int unit = seg ? unit1 : unit0, s_begin = seg ? 0 : b0, s_end = seg ? e1 : e0;
    const int pass = unit / plan.pblocks, pb = unit % plan.pblocks;
    const int p0_raw = pb * DQ_COLS_WG + wave * 32;
    const bool pvalid = p0_raw < N;          // N is a multiple of 128: valid waves come in groups of four
    const int p0 = pvalid ? p0_raw : N - 32;  // idle waves re-read the last group, never store

    // Code words: lane (column c, k-tile kt, half h) reads words 2c + h and
    // 2c + h + 1 (mod 32) of tile (2 s + kt, (p0 + 16 f) / 16).
    const int c = lane & 15, kt = lane >> 5, h = (lane >> 4) & 1;
    const int d = 2 * c + h;
    const uint32_t row_bytes = (uint32_t)ldt * 128;  // one k-tile row of codes
    uint32_t voff[2][2];
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const int nt = (p0 + 16 * f) / 16;
      voff[f][0] = (uint32_t)(kt * row_bytes + nt * 128 + 4 * d);
      voff[f][1] = (uint32_t)(kt * row_bytes + nt * 128 + 4 * ((d + 1) & 31));
    }
    const __amdgpu_buffer_rsrc_t crs = make_rsrc(codes, (uint32_t)((int64_t)K * ldt * 8));
    constexpr int kCodeLoads = 4;  // VMEM loads per call of load_codes
    auto load_codes = [&](int s, uint32_t (&w)[2][2]) {
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int j = 0; j < 2; ++j) w[f][j] = buffer_load_u32(crs, voff[f][j], (uint32_t)(2 * s) * row_bytes);
    };

    // x stage: SPB consecutive 32-k steps of the pass's NQ row fragments (16
    // rows x 32 k each), fragment f = j NQ + qt for step j of the stage and row
    // fragment qt, clamped to the last fragment of the padded rows (rows past M
    // are zero or repeats and are never stored); wave w loads fragments 2 w
    // and 2 w + 1, which belong to one step. Buffer loads (a fixed lane
    // offset, the step in the scalar offset): no 64-bit address registers to
    // rebuild while code-word loads are in flight.
    const int nq16 = (M + 31) / 32 * 2, q16_0 = pass * NQ;
    const __amdgpu_buffer_rsrc_t xrs =
        make_rsrc(xf + (int64_t)q16_0 * ks32 * 512, (uint32_t)(min(NQ, nq16 - q16_0) * ks32 * 1024));
    const int xj = (2 * wave) / NQ;  // the step of the stage this wave's fragments belong to
    uint32_t xoff[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
      xoff[i] = (uint32_t)((min(q16_0 + (2 * wave + i) % NQ, nq16 - 1) - q16_0) * ks32 * 1024 + 16 * lane);
    auto load_x = [&](int s0, int buf) {  // the stage of steps s0 .. s0 + SPB - 1
#pragma unroll
      for (int i = 0; i < 2; ++i)
        dq_buffer_load_lds16(xrs, (dq_lds_void*)(xs + buf * XSTAGE + (2 * wave + i) * 512), xoff[i],
                             (uint32_t)(s0 + xj) * 1024);
    };
    auto xfrag = [&](int buf, int j, int qt) {
      return *reinterpret_cast<const f16x8*>(xs + buf * XSTAGE + (j * NQ + qt) * 512 + 8 * lane);
    };

    f32x4 acc[2][NQ];
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int qt = 0; qt < NQ; ++qt) acc[f][qt] = (f32x4){0.f, 0.f, 0.f, 0.f};

    // Rings: code words of steps s .. s + 3; the codebook reads of step s + 1
    // are issued during step s.
    uint32_t wr[4][2][2];
#pragma unroll
    for (int u = 0; u < 4; ++u) load_codes(min(s_begin + u, s_end - 1), wr[u]);
    load_x(s_begin, 0);
    load_x(min(s_begin + SPB, s_end - SPB), 1);
    __builtin_amdgcn_s_waitcnt(0);  // the codebook, the first code words and both x stages have landed
    __syncthreads();
    uint32_t g[2][8];
    dq_gather(cb_lds, wr[0][0], g[0]);
    dq_gather(cb_lds, wr[0][1], g[1]);

    // Step s, phase u = (s - s_begin) % UL: code-word ring slot u % 4, x
    // buffer (u / SPB) % 2, step u % SPB of its stage. NQ slots, each the 2
    // MFMAs of one row fragment plus one piece of the next step's work in
    // source order fenced by scheduling barriers: the x fragment kXAhead slots
    // ahead, (slot kCodeSlot) the code words of s + 4, and (slots
    // kGatherSlot..NQ - 1, evenly) the 8 codebook read pairs of s + 1. After
    // the last step of a stage, one barrier and the loads of the stage after
    // next. Measured at M = 256..2048 on both MLP geometries with 16
    // fragments: fragments 6 ahead and the reads in the second half beat 2
    // ahead and the first half by 2-4 %; staggering the halves between the two
    // waves of a SIMD, or one read pair per slot, did not help. Stages of
    // several steps keep the barriers of the short passes (4 and 8 fragments)
    // to one per 16 fragments.
    constexpr int kXAhead = NQ < 6 ? NQ : 6, kCodeSlot = NQ >= 8 ? 4 : 1, kGatherSlot = NQ == 16 ? 8 : 0;
    constexpr int kGatherPerSlot = 8 / (NQ - kGatherSlot);
    constexpr int UL = SPB > 2 ? 2 * SPB : 4;  // steps per unrolled block: whole stages and ring turns
    static_assert(kGatherPerSlot * (NQ - kGatherSlot) == 8, "all 8 codebook read pairs of the next step are issued");
    static_assert(kCodeSlot < NQ && kXAhead <= NQ, "slot numbers");
    static_assert(UL % 4 == 0 && UL % (2 * SPB) == 0, "an unrolled block is whole ring turns and stage pairs");
    auto step = [&](auto U, int s) {
      constexpr int u = decltype(U)::value, b = (u / SPB) & 1, j = u % SPB, ur = u & 3;
      const int s4 = min(s + 4, s_end - 1);
      const f16x8 a0 = dq_pack(g[0]), a1 = dq_pack(g[1]);
      uint32_t off[2][8];
      window_offsets8(wr[(ur + 1) & 3][0][0], wr[(ur + 1) & 3][0][1], off[0]);
      window_offsets8(wr[(ur + 1) & 3][1][0], wr[(ur + 1) & 3][1][1], off[1]);
      f16x8 xq[kXAhead + 1];
#pragma unroll
      for (int i = 0; i < kXAhead; ++i) xq[i] = xfrag(b, j, i);
#pragma unroll
      for (int qt = 0; qt < NQ; ++qt) {
        if (qt + kXAhead < NQ) xq[(qt + kXAhead) % (kXAhead + 1)] = xfrag(b, j, qt + kXAhead);
        acc[0][qt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, xq[qt % (kXAhead + 1)], acc[0][qt], 0, 0, 0);
        acc[1][qt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, xq[qt % (kXAhead + 1)], acc[1][qt], 0, 0, 0);
        if (qt >= kGatherSlot) {
#pragma unroll
          for (int i = 0; i < kGatherPerSlot; ++i) {
            const int jj = (qt - kGatherSlot) * kGatherPerSlot + i;
            g[0][jj] = lds_cb(cb_lds, off[0][jj]);
            g[1][jj] = lds_cb(cb_lds, off[1][jj]);
          }
        }
        if (qt == kCodeSlot) load_codes(s4, wr[ur]);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (j == SPB - 1) {
        // every wave is done with x buffer b and its loads of the next stage
        // (issued before this stage's SPB x kCodeLoads code-word loads) have
        // landed; then the stage after next goes into buffer b
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(SPB * kCodeLoads) : "memory");
        __syncthreads();
        load_x(min(s + 1 + SPB, s_end - SPB), b);
      }
    };
    // every k range is a whole number of half blocks (UL / 2 steps: the plan
    // cuts K in multiples of 2 SPB 16-k steps, and K / 32 is a multiple of 4)
    auto block = [&](int s, auto... us) { (step(us, s + decltype(us)::value), ...); };
    auto half_block = [&](int s) {
      if constexpr (UL == 4)
        block(s, std::integral_constant<int, 0>{}, std::integral_constant<int, 1>{});
      else
        block(s, std::integral_constant<int, 0>{}, std::integral_constant<int, 1>{}, std::integral_constant<int, 2>{},
              std::integral_constant<int, 3>{});
    };
    int s = s_begin;
    for (; s + UL - 1 < s_end; s += UL) {
      if constexpr (UL == 4)
        block(s, std::integral_constant<int, 0>{}, std::integral_constant<int, 1>{}, std::integral_constant<int, 2>{},
              std::integral_constant<int, 3>{});
      else
        block(s, std::integral_constant<int, 0>{}, std::integral_constant<int, 1>{}, std::integral_constant<int, 2>{},
              std::integral_constant<int, 3>{}, std::integral_constant<int, 4>{}, std::integral_constant<int, 5>{},
              std::integral_constant<int, 6>{}, std::integral_constant<int, 7>{});
    }
    if (s < s_end) half_block(s);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the last (repeated) loads land before the LDS is reused
    __syncthreads();

    // Lane holds D[p = p0 + 16 f + 4 (lane >> 4) + r][q = 16 qt + (lane & 15)].
    const int pl = 4 * (lane >> 4), ql = lane & 15;
    if (TAIL) {
      // partials[slot][q][p] over the unit's R rows and 256 columns; slot: the
      // workgroup, or (stream-K) workgroup + tail unit, distinct for every
      // (run, unit) pair since consecutive runs move on by at least one in
      // one of the two
      if (pvalid) {
        const int slot = (int)blockIdx.x + (plan.sk_steps ? unit - plan.full : 0);
        float* base = partials + (int64_t)slot * R * DQ_COLS_WG + wave * 32 + pl;
#pragma unroll
        for (int qt = 0; qt < NQ; ++qt)
#pragma unroll
          for (int f = 0; f < 2; ++f)
            *reinterpret_cast<f32x4*>(base + (16 * qt + ql) * DQ_COLS_WG + 16 * f) = acc[f][qt];
      }
      continue;
    }

    // A whole unit: column scales into the accumulators, then rounds of RR
    // rows through the LDS (fp32 [row][256 columns], up to 128 KiB, where the
    // codebook was): 16 lanes per (row, 128-column block) read 8 consecutive
    // columns, rotate (the arithmetic of the decode path's output stage),
    // apply the signs and store fp16 y.
    constexpr int RR = R < 128 ? R : 128, QR = RR / 16;
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const u32x2 sc = *reinterpret_cast<const u32x2*>(scale + p0 + 16 * f + pl);
      const float s0 = bits_lo_f16(sc[0]), s1 = bits_hi_f16(sc[0]), s2 = bits_lo_f16(sc[1]), s3 = bits_hi_f16(sc[1]);
#pragma unroll
      for (int qt = 0; qt < NQ; ++qt) {
        acc[f][qt][0] *= s0;
        acc[f][qt][1] *= s1;
        acc[f][qt][2] *= s2;
        acc[f][qt][3] *= s3;
      }
    }
    float* tb = reinterpret_cast<float*>(lds);
    const uint32_t smask = sign_n ? 0x80008000u : 0u;
#pragma unroll
    for (int rnd = 0; rnd < R / RR; ++rnd) {
      if (pvalid)
#pragma unroll
        for (int qt = 0; qt < QR; ++qt)
#pragma unroll
          for (int f = 0; f < 2; ++f)
            *reinterpret_cast<f32x4*>(tb + (16 * qt + ql) * DQ_COLS_WG + wave * 32 + 16 * f + pl) =
                acc[f][QR * rnd + qt];
      __syncthreads();
      // RR rows x 2 blocks x 16 lanes = 32 RR lane tasks, RR / 16 per thread
      const int q16 = threadIdx.x & 15;
#pragma unroll
      for (int i = 0; i < RR / 16; ++i) {
        const int item = (threadIdx.x >> 4) + 32 * i;  // (row, block)
        const int r = item >> 1, blk = item & 1;
        const int row = pass * R + RR * rnd + r;
        const int col0 = pb * DQ_COLS_WG + 128 * blk;
        const f32x4* src = reinterpret_cast<const f32x4*>(tb + r * DQ_COLS_WG + 128 * blk + 8 * q16);
        const f32x4 v0 = src[0], v1 = src[1];
        float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        wht128_16(v, q16);
        if (row < M && col0 < N) {  // uniform over the 16 lanes
          const int col = col0 + 8 * q16;
          const u32x4 sg = *reinterpret_cast<const u32x4*>((sign_n ? sign_n : scale) + col);
          u32x4 o;
#pragma unroll
          for (int j = 0; j < 4; ++j) o[j] = pack_f16x2(v[2 * j] * EXL3_INV_SQRT128, v[2 * j + 1] * EXL3_INV_SQRT128);
          o ^= sg & smask;
          *reinterpret_cast<u32x4*>(y + (int64_t)row * ldy + col) = o;
        }
      }
      __syncthreads();  // the buffer is rewritten in the next round
    }
  }  // segments
}

// Sums the tail pieces of one unit in k order, applies the column scales,
// the output rotation and the signs, and stores fp16 y: 16 lanes per (unit,
// row, 128-column block), 8 columns per lane (the arithmetic of the decode
// path's output stage).
__global__ __launch_bounds__(256) void dq_fixup_kernel(const float* __restrict__ partials, int32_t R, DqPlan plan,
                                                       const uint16_t* __restrict__ scale,
                                                       const uint16_t* __restrict__ sign_n, uint16_t* __restrict__ y,
                                                       int64_t ldy, int32_t M, int32_t N, int32_t K) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int q = (int)(gid & 15);
  const int64_t item = gid >> 4;  // (tail unit, row, block)
  const int64_t nitems = (int64_t)plan.tail * R * 2;
  const int64_t it = item < nitems ? item : nitems - 1;
  const int t = (int)(it / (2 * R)), r = (int)((it / 2) % R), b = (int)(it % 2);
  const int unit = plan.full + t, pass = unit / plan.pblocks, pb = unit % plan.pblocks;
  const int row = pass * R + r;
  const int col0 = pb * DQ_COLS_WG + 128 * b;  // a multiple of 128: inside N or wholly past it
  const bool ok = item < nitems && row < M && col0 < N;
  const int col = min(col0, N - 128) + 8 * q;
  const u32x4 sc = *reinterpret_cast<const u32x4*>(scale + col);
  const u32x4 sg = *reinterpret_cast<const u32x4*>((sign_n ? sign_n : scale) + col);
  const uint32_t smask = sign_n ? 0x80008000u : 0u;
  // the unit's pieces in k order: slots t tail_ks .. + tail_ks - 1, or
  // (stream-K) the runs v that overlap the unit's steps [t ks32, (t + 1)
  // ks32), slot v + t
  const int64_t piece = (int64_t)R * DQ_COLS_WG / 4;  // f32x4 per slot
  const f32x4* src0 = reinterpret_cast<const f32x4*>(partials + (int64_t)r * DQ_COLS_WG + 128 * b + 8 * q);
  const int ks32 = K / 32;
  int v_lo = t * plan.tail_ks, v_hi = v_lo + plan.tail_ks - 1;
  if (plan.sk_steps) {
    v_lo = (int)((int64_t)t * ks32 / plan.sk_steps);
    v_hi = (int)(((int64_t)(t + 1) * ks32 - 1) / plan.sk_steps);
  }
  auto slot = [&](int v) { return plan.sk_steps ? v + t : v; };
  float v[8];
  {
    const f32x4* src = src0 + slot(v_lo) * piece;
    const f32x4 p0 = src[0], p1 = src[1];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = p0[j];
      v[4 + j] = p1[j];
    }
  }
  for (int w = v_lo + 1; w <= v_hi; ++w) {
    const f32x4* src = src0 + slot(w) * piece;
    const f32x4 p0 = src[0], p1 = src[1];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] += p0[j];
      v[4 + j] += p1[j];
    }
  }
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
  if (ok) *reinterpret_cast<u32x4*>(y + (int64_t)row * ldy + col) = o;
}

// The eight-wave dequant-GEMM: passes of R = 32 * plan.nqb rows (nqb 2, 4 or
// 8: NQ = 2 nqb row fragments of 16), whole units, then k-split pieces and
// their fixup.
hipError_t launch_dqgemm2(const uint16_t* xf16, const uint32_t* codes, const uint16_t* cb, const uint16_t* scale,
                          const uint16_t* sign_n, uint16_t* y, int64_t ldy, float* partials, int32_t K, int32_t N,
                          int32_t ldt, int32_t M, const DqPlan& plan, hipStream_t stream) {
  if (plan.nqb != 2 && plan.nqb != 4 && plan.nqb != 8) return hipErrorInvalidValue;
#define EXL3_DQ2_LAUNCH(nq, tail, grid)                                                                         \
  dqgemm2_kernel<nq, tail><<<(grid), DQ2_THREADS, 0, stream>>>(xf16, codes, cb, scale, sign_n, y, ldy, partials, K, \
                                                               N, ldt, M, plan)
#define EXL3_DQ2_LAUNCH_NQ(tail, grid)    \
  switch (plan.nqb) {                      \
    case 2:                                \
      EXL3_DQ2_LAUNCH(4, tail, grid);      \
      break;                               \
    case 4:                                \
      EXL3_DQ2_LAUNCH(8, tail, grid);      \
      break;                               \
    default:                               \
      EXL3_DQ2_LAUNCH(16, tail, grid);     \
  }
  if (plan.full > 0) EXL3_DQ2_LAUNCH_NQ(false, plan.full)
  if (plan.tail > 0) EXL3_DQ2_LAUNCH_NQ(true, plan.sk_steps ? plan.sk_wgs : plan.tail * plan.tail_ks)
#undef EXL3_DQ2_LAUNCH_NQ
#undef EXL3_DQ2_LAUNCH
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || plan.tail == 0) return e;
  const int R = 32 * plan.nqb;
  const int64_t threads = (int64_t)plan.tail * R * 2 * 16;
  dq_fixup_kernel<<<(unsigned)((threads + 255) / 256), 256, 0, stream>>>(partials, R, plan, scale, sign_n, y, ldy, M,
                                                                          N, K);
  return hipGetLastError();
}

size_t dq_partial_bytes(const DqPlan& plan) {
  const size_t slots = plan.sk_steps ? (size_t)plan.sk_wgs + plan.tail - 1 : (size_t)plan.tail * plan.tail_ks;
  return slots * 32 * plan.nqb * DQ_COLS_WG * sizeof(float);
}

hipError_t launch_dqgemm(const uint16_t* xf, const uint32_t* codes, const uint16_t* cb, const uint16_t* scale,
                         const uint16_t* sign_n, uint16_t* y, int64_t ldy, float* partials, int32_t K, int32_t N,
                         int32_t ldt, int32_t M, const DqPlan& plan, hipStream_t stream) {
#define EXL3_DQ_LAUNCH(nqb, tail, grid)                                                                    \
  dqgemm_kernel<nqb, tail><<<grid, DQ_THREADS, 0, stream>>>(xf, codes, cb, scale, sign_n, y, ldy, partials, K, N, \
                                                            ldt, M, plan)
#define EXL3_DQ_CASE(nqb)                                                                     \
  case nqb:                                                                                   \
    if (plan.full > 0) EXL3_DQ_LAUNCH(nqb, false, plan.full);                                 \
    if (plan.tail > 0) EXL3_DQ_LAUNCH(nqb, true, plan.tail * plan.tail_ks);                   \
    break;
  switch (plan.nqb) {
    EXL3_DQ_CASE(1)
    EXL3_DQ_CASE(2)
    EXL3_DQ_CASE(4)
    EXL3_DQ_CASE(8)
    default:
      return hipErrorInvalidValue;
  }
#undef EXL3_DQ_CASE
#undef EXL3_DQ_LAUNCH
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || plan.tail == 0) return e;
  const int R = 32 * plan.nqb;
  const int64_t threads = (int64_t)plan.tail * R * 2 * 16;
  dq_fixup_kernel<<<(unsigned)((threads + 255) / 256), 256, 0, stream>>>(partials, R, plan, scale, sign_n, y, ldy, M,
                                                                          N, K);
  return hipGetLastError();
}

}  // namespace exl3
