// Trellis -> fp16 weight reconstruction (vLLM PR #316, "Kernel measurements":
// reconstruct / reconstruct_slice; "Change": one reused fp16 scratch of at
// most 32768 columns).
//
// Per weight: 0.5 byte of codes read, 2 bytes of fp16 written, one random
// 16-bit gather from the 128 KiB codebook held in LDS. The kernels are
// persistent (one 128 KiB codebook copy per workgroup, one workgroup per CU)
// and each lane decodes one whole tile column: 16 consecutive k for one n, the
// natural run of the k-fastest trellis.
#include "common.h"
#include "trellis.h"

namespace exl3 {

// Tile column c of a tile: steps 16c .. 16c+15 are the 16-bit windows at
// bits BITS (16c + r), r = 0..15, as codebook byte offsets. At 4 bits they lie
// inside words 2c, 2c+1 and (2c+2) mod 32.
template <int BITS>
__device__ __forceinline__ void tile_column_offsets(const uint32_t* __restrict__ tile, int c,
                                                    uint32_t (&off)[16]) {
  if constexpr (BITS == 4) {
    const uint32_t w0 = tile[2 * c], w1 = tile[2 * c + 1], w2 = tile[(2 * c + 2) & 31];
    uint32_t a[8], b[8];
    window_offsets8(w0, w1, a);
    window_offsets8(w1, w2, b);
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      off[r] = a[r];
      off[8 + r] = b[r];
    }
  } else {
    constexpr int NW = TrellisWidth<BITS>::words(16, 16);
    const int start = 16 * BITS * c;
    uint32_t w[NW];
#pragma unroll
    for (int j = 0; j < NW; ++j) w[j] = tile[(start / 32 + j) % (8 * BITS)];
    window_offsets_any<BITS, 16, NW>(w, (uint32_t)(start & 31), off);
  }
}

// Writes W^T: wt[j * ldw + k] = W[k][16 nt0 + j], j < 16 n_nt.
// A unit is 4 k-tiles x 1 n-tile: lane (c = lane >> 2, dk = lane & 3) decodes
// column c of k-tile 4 kg + dk, i.e. the 32 bytes at k offset 32 dk of the
// unit's 128-byte piece of W^T row c. The quad of lanes holding one row swaps
// halves with two DPP transposes, so each 16-byte store instruction writes 64
// contiguous bytes of 16 rows (not 16-byte pieces 32 bytes apart).
//
// Reads and writes are kept apart in time: each wave first issues the loads
// of the code words and scales of all its units, at most RcWidth::kRmax, held
// in registers, and only then decodes and stores them, with no wait on the
// vector-memory counter. Over the chip the reads of a launch run before its
// writes instead of interleaved with them: HBM serves the mix of 178 MB
// written and 44.5 MB read of a 4-bit K5120 x N17408 slice at 5.5 TB/s this
// way and at 3.4 TB/s interleaved. At 4 bits a lane loads two words per unit
// (one dwordx2: words 2c, 2c+1; word 2c+2 is the next column's first word,
// taken with one ds_bpermute); at other widths it loads its column's whole
// word span. A launch covers at most kRmax units per wave of a full grid;
// larger slices take several launches.
#define RC_WAVES 8
#define RC_GROUP 2

template <int BITS>
struct RcWidth {
  static constexpr int kWords = BITS == 4 ? 2 : TrellisWidth<BITS>::words(16, 16);  // code words per unit
  // units per wave per launch: about 132 registers of words and scales
  static constexpr int kRmax = (132 / (kWords + 1)) & ~(RC_GROUP - 1);
};

template <int BITS>
__global__ __launch_bounds__(64 * RC_WAVES) void reconstruct_nk_kernel(const uint32_t* __restrict__ codes,
                                                                       const uint16_t* __restrict__ cb,
                                                                       const uint16_t* __restrict__ scale,
                                                                       int32_t K, int32_t N, int32_t nt0,
                                                                       int32_t n_nt, uint16_t* __restrict__ wt,
                                                                       int64_t ldw, int32_t unit0, int32_t units) {
  constexpr int RMAX = RcWidth<BITS>::kRmax, NW = RcWidth<BITS>::kWords;
  constexpr uint32_t TB = TrellisWidth<BITS>::kTileBytes;
  __shared__ uint16_t cb_lds[65536];
  const int lane = threadIdx.x & 63;
  const int c = lane >> 2, dk = lane & 3;
  const int tiles_n = N / 16;
  const int nwaves = gridDim.x * RC_WAVES;
  const int wv = blockIdx.x * RC_WAVES + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // this wave's units: unit0 + wv, + nwaves, ... (at most RMAX of them)
  const int my = wv < units ? (units - 1 - wv) / nwaves + 1 : 0;
  const int u0 = unit0 + wv;
  const int dq = nwaves / n_nt, dr = nwaves % n_nt;

  const __amdgpu_buffer_rsrc_t crs = make_rsrc(codes, (uint32_t)((int64_t)K * N * BITS / 8));
  // byte offsets of the lane's words inside its unit: k-tile 4 kg + dk, the
  // words of column c from word (16 c BITS) / 32 on, wrapping in the tile
  const int start = 16 * BITS * c;
  uint32_t vw[NW];
#pragma unroll
  for (int j = 0; j < NW; ++j) vw[j] = (uint32_t)dk * tiles_n * TB + 4u * ((start / 32 + j) % (8 * BITS));
  const __amdgpu_buffer_rsrc_t srs = make_rsrc(scale, (uint32_t)N * 2);
  const uint32_t vsc = 4u * (c >> 1), sc_shift = 16u * (c & 1);
  const int src4 = ((lane + 4) & 63) * 4;  // 4 bits: lane holding word (2c + 2) mod 32 as its first word

  uint32_t cw[RMAX][NW];
  uint32_t sc[RMAX];
  // Loads of all units (wave-uniform guards).
  {
    int kg = u0 / n_nt, ntl = u0 % n_nt;
#pragma unroll
    for (int i = 0; i < RMAX; ++i) {
      if (i < my) {
        const uint32_t so = (uint32_t)(4 * kg * tiles_n + nt0 + ntl) * TB;
        if constexpr (BITS == 4) {
          const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(crs, vw[0], so, 0);
          cw[i][0] = v[0];
          cw[i][1] = v[1];
        } else {
#pragma unroll
          for (int j = 0; j < NW; ++j) cw[i][j] = buffer_load_u32(crs, vw[j], so);
        }
        sc[i] = buffer_load_u32(srs, vsc, (uint32_t)(32 * (nt0 + ntl)));
      }
      kg += dq;
      ntl += dr;
      if (ntl >= n_nt) {
        ntl -= n_nt;
        ++kg;
      }
    }
  }
  load_codebook<64 * RC_WAVES>(cb_lds, cb);
  __syncthreads();
  if (my == 0) return;  // no workgroup barrier follows

  // Decode RC_GROUP units at a time: all their gathers are issued before the
  // first is used.
  int kg_d = u0 / n_nt, ntl_d = u0 % n_nt;  // unit being decoded
#pragma unroll
  for (int i0 = 0; i0 < RMAX; i0 += RC_GROUP) {
    if (i0 < my) {
      uint32_t g[RC_GROUP][16];
#pragma unroll
      for (int i = 0; i < RC_GROUP; ++i) {
        uint32_t off[16];
        if constexpr (BITS == 4) {
          const uint32_t w0 = cw[i0 + i][0], w1 = cw[i0 + i][1];
          const uint32_t w2 = (uint32_t)__builtin_amdgcn_ds_bpermute(src4, (int)w0);
          uint32_t a[8], b[8];
          window_offsets8(w0, w1, a);
          window_offsets8(w1, w2, b);
#pragma unroll
          for (int r = 0; r < 8; ++r) {
            off[r] = a[r];
            off[8 + r] = b[r];
          }
        } else {
          window_offsets_any<BITS, 16, NW>(cw[i0 + i], (uint32_t)(start & 31), off);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) g[i][r] = lds_cb(cb_lds, off[r]);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < RC_GROUP; ++i) {
        const int kg = kg_d, ntl = ntl_d;
        kg_d += dq;
        ntl_d += dr;
        if (ntl_d >= n_nt) {
          ntl_d -= n_nt;
          ++kg_d;
        }
        if (i0 + i >= my) break;  // uniform
        const f16 s = __builtin_bit_cast(f16, (uint16_t)(sc[i0 + i] >> sc_shift));
        const f16x2 s2 = {s, s};
        u32x4 o[2];  // 16-byte pieces 2 dk and 2 dk + 1 of the row's 128 bytes
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          f16x2 v = {__builtin_bit_cast(f16, (uint16_t)g[i][2 * j]),
                     __builtin_bit_cast(f16, (uint16_t)g[i][2 * j + 1])};
          v = v * s2;  // one fp16 rounding of the exact product
          o[j >> 2][j & 3] = __builtin_bit_cast(uint32_t, v);
        }
        // lane dk of the quad stores piece dk, then piece 4 + dk: piece p
        // lives in lane p >> 1 as o[p & 1]
        u32x4 lo, hi;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t l0 = dpp_mov_u32<EXL3_DPP_PAIR_LO>(o[0][e]), l1 = dpp_mov_u32<EXL3_DPP_PAIR_LO>(o[1][e]);
          const uint32_t h0 = dpp_mov_u32<EXL3_DPP_PAIR_HI>(o[0][e]), h1 = dpp_mov_u32<EXL3_DPP_PAIR_HI>(o[1][e]);
          lo[e] = (dk & 1) ? l1 : l0;
          hi[e] = (dk & 1) ? h1 : h0;
        }
        uint16_t* row = wt + (int64_t)(16 * ntl + c) * ldw + 64 * kg;
        *reinterpret_cast<u32x4*>(row + 8 * dk) = lo;
        *reinterpret_cast<u32x4*>(row + 32 + 8 * dk) = hi;
      }
    }
  }
}

// Writes W (canonical K x n layout) or the raw states, through an LDS
// transpose: each wave decodes 1 k-tile x 4 n-tiles, stages the 16 x 64 block
// in LDS, and writes 16 rows of 128 contiguous bytes.
template <bool STATES, int BITS>
__global__ __launch_bounds__(512) void reconstruct_kn_kernel(const uint32_t* __restrict__ codes,
                                                             const uint16_t* __restrict__ cb,
                                                             const uint16_t* __restrict__ scale, int32_t K,
                                                             int32_t N, int32_t nt0, int32_t n_nt,
                                                             uint16_t* __restrict__ w, int64_t ldw) {
  __shared__ uint16_t cb_lds[STATES ? 8 : 65536];
  __shared__ uint16_t stage[8][16][64];
  if (!STATES) load_codebook<512>(cb_lds, cb);
  __syncthreads();

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int tiles_n = N / 16;
  const int n_ng = (n_nt + 3) / 4;
  const int64_t units = (int64_t)(K / 16) * n_ng;
  for (int64_t base = (int64_t)blockIdx.x * 8; base < units; base += (int64_t)gridDim.x * 8) {
    const int64_t u = base + wave;
    const bool active = u < units;
    const int kt = active ? (int)(u / n_ng) : 0;
    const int ng = active ? (int)(u % n_ng) : 0;
    const int ntl = 4 * ng + (lane >> 4);
    const int c = lane & 15;
    uint16_t vals[16];
    if (active && ntl < n_nt) {
      const int nt = nt0 + ntl;
      const uint32_t* tile = codes + ((int64_t)kt * tiles_n + nt) * TrellisWidth<BITS>::kTileWords;
      uint32_t off[16];
      tile_column_offsets<BITS>(tile, c, off);
      if (STATES) {
#pragma unroll
        for (int r = 0; r < 16; ++r) vals[r] = (uint16_t)(off[r] >> 1);
      } else {
        const f16 s = __builtin_bit_cast(f16, scale[16 * nt + c]);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          f16 v = __builtin_bit_cast(f16, lds_cb(cb_lds, off[r])) * s;
          vals[r] = __builtin_bit_cast(uint16_t, v);
        }
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) vals[r] = 0;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) stage[wave][r][lane] = vals[r];
    __syncthreads();
    const int r = lane >> 2, part = lane & 3;
    const u32x4* src = reinterpret_cast<const u32x4*>(&stage[wave][r][16 * part]);
    const u32x4 v0 = src[0], v1 = src[1];
    if (active && 4 * ng + part < n_nt) {
      u32x4* dst = reinterpret_cast<u32x4*>(w + (int64_t)(16 * kt + r) * ldw + 64 * ng + 16 * part);
      dst[0] = v0;
      dst[1] = v1;
    }
    __syncthreads();
  }
}

static int persistent_grid(int64_t units, int units_per_block) {
  int64_t g = (units + units_per_block - 1) / units_per_block;
  return (int)(g < 256 ? (g < 1 ? 1 : g) : 256);
}

template <int BITS>
static hipError_t launch_reconstruct_nk_w(const uint32_t* codes, const uint16_t* cb, const uint16_t* scale, int32_t K,
                                          int32_t N, int32_t n0, int32_t n_nt, uint16_t* wt, int64_t ldw,
                                          hipStream_t stream) {
  // the fewest launches of at most kRmax units per wave of a full grid, with
  // the units spread evenly over them
  const int32_t units = (K / 64) * n_nt;
  const int32_t per_launch = 256 * RC_WAVES * RcWidth<BITS>::kRmax;
  const int32_t launches = (units + per_launch - 1) / per_launch;
  const int32_t each = (units + launches - 1) / launches;
  for (int32_t u0 = 0; u0 < units; u0 += each) {
    const int32_t n = units - u0 < each ? units - u0 : each;
    const int grid = persistent_grid(n, RC_WAVES);
    reconstruct_nk_kernel<BITS>
        <<<grid, 64 * RC_WAVES, 0, stream>>>(codes, cb, scale, K, N, n0 / 16, n_nt, wt, ldw, u0, n);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_reconstruct_nk(const uint32_t* codes, const uint16_t* cb, const uint16_t* scale, int32_t K,
                                 int32_t N, int32_t bits, int32_t n0, int32_t n_count, uint16_t* wt, int64_t ldw,
                                 hipStream_t stream) {
  const int n_nt = n_count / 16;
  if (n_nt == 0) return hipSuccess;
  switch (bits) {
#define EXL3_RC_NK(b) \
  case b:             \
    return launch_reconstruct_nk_w<b>(codes, cb, scale, K, N, n0, n_nt, wt, ldw, stream);
    EXL3_RC_NK(1) EXL3_RC_NK(2) EXL3_RC_NK(3) EXL3_RC_NK(4) EXL3_RC_NK(5) EXL3_RC_NK(6) EXL3_RC_NK(7) EXL3_RC_NK(8)
#undef EXL3_RC_NK
    default:
      return hipErrorInvalidValue;
  }
}

hipError_t launch_reconstruct_kn(const uint32_t* codes, const uint16_t* cb, const uint16_t* scale, int32_t K,
                                 int32_t N, int32_t bits, int32_t n0, int32_t n_count, uint16_t* w, int64_t ldw,
                                 bool states, hipStream_t stream) {
  const int n_nt = n_count / 16;
  if (n_nt == 0) return hipSuccess;
  const int grid = persistent_grid((int64_t)(K / 16) * ((n_nt + 3) / 4), 8);
  switch (bits) {
#define EXL3_RC_KN(b)                                                                                            \
  case b:                                                                                                        \
    if (states)                                                                                                  \
      reconstruct_kn_kernel<true, b><<<grid, 512, 0, stream>>>(codes, cb, scale, K, N, n0 / 16, n_nt, w, ldw); \
    else                                                                                                         \
      reconstruct_kn_kernel<false, b><<<grid, 512, 0, stream>>>(codes, cb, scale, K, N, n0 / 16, n_nt, w, ldw); \
    break;
    EXL3_RC_KN(1) EXL3_RC_KN(2) EXL3_RC_KN(3) EXL3_RC_KN(4) EXL3_RC_KN(5) EXL3_RC_KN(6) EXL3_RC_KN(7) EXL3_RC_KN(8)
#undef EXL3_RC_KN
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace exl3
