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

// Tile column c of tile (kt, nt): steps 16c .. 16c+15 are the 16-bit windows
// at bits 64c + 4r, r = 0..15, i.e. inside words 2c, 2c+1 and (2c+2) mod 32.
__device__ __forceinline__ void tile_column_offsets(const uint32_t* __restrict__ tile, int c,
                                                    uint32_t (&off)[16]) {
  const uint32_t w0 = tile[2 * c], w1 = tile[2 * c + 1], w2 = tile[(2 * c + 2) & 31];
  uint32_t a[8], b[8];
  window_offsets8(w0, w1, a);
  window_offsets8(w1, w2, b);
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    off[r] = a[r];
    off[8 + r] = b[r];
  }
}

// Writes W^T: wt[j * ldw + k] = W[k][16 nt0 + j], j < 16 n_nt.
// A unit is 4 k-tiles x 1 n-tile: lane (c = lane >> 2, dk = lane & 3) decodes
// column c of k-tile 4 kg + dk, i.e. the 32 bytes at k offset 32 dk of the
// unit's 128-byte piece of W^T row c. The quad of lanes holding one row swaps
// halves with two DPP transposes, so each 16-byte store instruction writes 64
// contiguous bytes of 16 rows (not 16-byte pieces 32 bytes apart). A wave
// walks its units (stride = all waves) in groups of RC_GROUP; the code words
// of the next group load into a second register set while the current group
// decodes, which keeps ~2 KB of codes per wave in flight.
#define RC_GROUP 4

struct RcRegs {
  uint32_t w0[RC_GROUP], w1[RC_GROUP], w2[RC_GROUP], sc[RC_GROUP];
};

__global__ __launch_bounds__(1024) void reconstruct_nk_kernel(const uint32_t* __restrict__ codes,
                                                              const uint16_t* __restrict__ cb,
                                                              const uint16_t* __restrict__ scale, int32_t K,
                                                              int32_t N, int32_t nt0, int32_t n_nt,
                                                              uint16_t* __restrict__ wt, int64_t ldw) {
  __shared__ uint16_t cb_lds[65536];
  load_codebook<1024>(cb_lds, cb);
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int c = lane >> 2, dk = lane & 3;
  const int tiles_n = N / 16;
  // Unit indices are wave-uniform 32-bit values (K / 64 * n_nt < 2^31 for any
  // K, N the layer accepts), so their arithmetic stays on the scalar unit.
  const int units = (K / 64) * n_nt;
  const int nwaves = gridDim.x * 16;
  int u = blockIdx.x * 16 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (u >= units) return;  // no workgroup barrier follows
  const int last = u + (units - 1 - u) / nwaves * nwaves;  // this wave's last unit

  const __amdgpu_buffer_rsrc_t crs = make_rsrc(codes, (uint32_t)((int64_t)K * N / 2));
  const uint32_t vrow = (uint32_t)dk * tiles_n * 128u;  // bytes from k-tile 4 kg to 4 kg + dk
  const uint32_t v0 = vrow + 8u * c, v1 = v0 + 4u, v2 = vrow + 4u * ((2 * c + 2) & 31);
  // scales: the aligned dword holding column 16 nt + c, then its half
  const __amdgpu_buffer_rsrc_t srs = make_rsrc(scale, (uint32_t)N * 2);
  const uint32_t vsc = 4u * (c >> 1), sc_shift = 16u * (c & 1);

  auto load_group = [&](int ug, RcRegs& R) {
#pragma unroll
    for (int i = 0; i < RC_GROUP; ++i) {
      const int uu = min(ug + i * nwaves, last);  // past the end: reload the last unit
      const int kg = uu / n_nt, ntl = uu % n_nt;
      const uint32_t so = (uint32_t)((4 * kg * tiles_n + nt0 + ntl) * 128);
      R.w0[i] = buffer_load_u32(crs, v0, so);
      R.w1[i] = buffer_load_u32(crs, v1, so);
      R.w2[i] = buffer_load_u32(crs, v2, so);
      R.sc[i] = buffer_load_u32(srs, vsc, (uint32_t)(32 * (nt0 + ntl)));
    }
  };
  // All RC_GROUP x 16 gathers of a group are issued before any is used, so a
  // wave keeps 64 codebook reads in flight. Units past the wave's last reuse
  // its last unit's words and store its (identical) bytes again: every group
  // issues the same 8 stores, which keeps the wait for the next group's code
  // words from also waiting on these stores (the vector-memory counter
  // covers both).
  auto decode_group = [&](int ug, const RcRegs& R) {
    uint32_t g[RC_GROUP][16];
#pragma unroll
    for (int i = 0; i < RC_GROUP; ++i) {
      uint32_t a[8], b[8];
      window_offsets8(R.w0[i], R.w1[i], a);
      window_offsets8(R.w1[i], R.w2[i], b);
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        g[i][r] = lds_cb(cb_lds, a[r]);
        g[i][8 + r] = lds_cb(cb_lds, b[r]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // keep every gather ahead of the first use
#pragma unroll
    for (int i = 0; i < RC_GROUP; ++i) {
      const int uu = min(ug + i * nwaves, last);
      const int kg = uu / n_nt, ntl = uu % n_nt;
      const f16 s = __builtin_bit_cast(f16, (uint16_t)(R.sc[i] >> sc_shift));
      const f16x2 s2 = {s, s};
      u32x4 o[2];  // 16-byte pieces 2 dk and 2 dk + 1 of the row's 128 bytes
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        f16x2 v = {__builtin_bit_cast(f16, (uint16_t)g[i][2 * j]), __builtin_bit_cast(f16, (uint16_t)g[i][2 * j + 1])};
        v = v * s2;  // one fp16 rounding of the exact product
        o[j >> 2][j & 3] = __builtin_bit_cast(uint32_t, v);
      }
      // lane dk of the quad stores piece dk, then piece 4 + dk: piece p lives
      // in lane p >> 1 as o[p & 1]
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
  };

  // Two register sets; every wait for a set's code words has the other set's
  // 8 stores and 16 loads behind it, on the first pass as in the loop.
  const int gstride = RC_GROUP * nwaves;
  RcRegs ra, rb;
  load_group(u, ra);
  load_group(u + gstride, rb);
  decode_group(u, ra);
  load_group(u + 2 * gstride, ra);
  for (int ub = u + gstride; ub <= last; ub += 2 * gstride) {
    decode_group(ub, rb);
    if (ub + gstride > last) break;
    load_group(ub + 2 * gstride, rb);
    decode_group(ub + gstride, ra);
    load_group(ub + 3 * gstride, ra);
  }
}

// Writes W (canonical K x n layout) or the raw states, through an LDS
// transpose: each wave decodes 1 k-tile x 4 n-tiles, stages the 16 x 64 block
// in LDS, and writes 16 rows of 128 contiguous bytes.
template <bool STATES>
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
      const uint32_t* tile = codes + ((int64_t)kt * tiles_n + nt) * 32;
      if (STATES) {
        const uint32_t w0 = tile[2 * c], w1 = tile[2 * c + 1], w2 = tile[(2 * c + 2) & 31];
        uint32_t a[8], b[8];
        window_states8(w0, w1, a);
        window_states8(w1, w2, b);
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          vals[r] = (uint16_t)a[r];
          vals[8 + r] = (uint16_t)b[r];
        }
      } else {
        uint32_t off[16];
        tile_column_offsets(tile, c, off);
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

hipError_t launch_reconstruct_nk(const uint32_t* codes, const uint16_t* cb, const uint16_t* scale, int32_t K,
                                 int32_t N, int32_t n0, int32_t n_count, uint16_t* wt, int64_t ldw,
                                 hipStream_t stream) {
  const int n_nt = n_count / 16;
  if (n_nt == 0) return hipSuccess;
  const int grid = persistent_grid((int64_t)(K / 64) * n_nt, 16);
  reconstruct_nk_kernel<<<grid, 1024, 0, stream>>>(codes, cb, scale, K, N, n0 / 16, n_nt, wt, ldw);
  return hipGetLastError();
}

hipError_t launch_reconstruct_kn(const uint32_t* codes, const uint16_t* cb, const uint16_t* scale, int32_t K,
                                 int32_t N, int32_t n0, int32_t n_count, uint16_t* w, int64_t ldw, bool states,
                                 hipStream_t stream) {
  const int n_nt = n_count / 16;
  if (n_nt == 0) return hipSuccess;
  const int grid = persistent_grid((int64_t)(K / 16) * ((n_nt + 3) / 4), 8);
  if (states)
    reconstruct_kn_kernel<true><<<grid, 512, 0, stream>>>(codes, cb, scale, K, N, n0 / 16, n_nt, w, ldw);
  else
    reconstruct_kn_kernel<false><<<grid, 512, 0, stream>>>(codes, cb, scale, K, N, n0 / 16, n_nt, w, ldw);
  return hipGetLastError();
}

}  // namespace exl3
