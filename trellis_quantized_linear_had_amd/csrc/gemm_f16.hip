// Dense fp16 GEMM with fp32 accumulation on the MFMA units, with the output
// rotation fused into the epilogue (vLLM PR #316, "Kernel measurements": the
// hgemm between the two had_r_128 calls; follow-up item 2: hgemm against
// torch.mm at the MLP shapes).
//
//   D[p][q] = sum_k A[p][k] * B[q][k]     A = W^T slice (P x K), B = Xr (Q x K)
//   y[q][n0 + p] = fp16(sign_n[n0 + p] * (1/sqrt128) * sum_{p'} H[p][p'] D[p'][q])
//
// Computing the transpose (p = output column n, q = input row m) puts the
// 128-column rotation along the MFMA's row dimension, which a lane holds in
// registers: six of its seven butterfly stages run in registers and one
// crosses lanes 32 apart.
//
// Tiling: 256 (p) x 256 (q) per workgroup, 64-wide k steps. Operands go from
// global memory straight into LDS (global_load_lds_dwordx4, no register
// staging), two stages, one barrier per k step. Inside a stage each 128-byte
// row is cut in 16-byte chunks XOR-swizzled by (row & 7), so the fragment
// reads (32 rows at one chunk) are bank-conflict free; the swizzle is applied
// on the global side, because a direct-to-LDS load writes lane i's 16 bytes at
// base + 16 i. 8 waves as 2 (p) x 4 (q), each 128 x 64 = 4 x 2
// v_mfma_f32_32x32x16_f16 tiles; two waves per SIMD hide each other's LDS and
// barrier waits.
//
// Workgroup order is XCD-aware: workgroups are dispatched round-robin over
// the 8 XCDs, so workgroup w is given tile (w % 8) * ceil(T / 8) + w / 8. Each
// XCD then walks a contiguous run of tiles, q fastest: the 8 q-tiles that
// share one 256-row strip of W^T run together on one XCD and read it through
// that XCD's L2.
#include "common.h"

namespace exl3 {

#define G_BP 256
#define G_BQ 256
#define G_BK 64
#define G_THREADS 512
#define G_STAGE (G_BP * G_BK + G_BQ * G_BK)  // halves per stage

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ int swz(int row, int chunk) { return row * G_BK + ((chunk ^ (row & 7)) << 3); }

// Per-lane byte offsets of the 4 x 16 bytes one wave loads per k step from
// 32 rows of a row-major operand (8 rows, 1 KB per instruction): row
// wave_row0 + 8 i + lane / 8, source chunk (lane % 8) ^ (row % 8). Rows past
// the end re-read the last row (never stored).
__device__ __forceinline__ void lane_offsets(int64_t ld, int row_base, int rows_valid, int wave_row0, int lane,
                                             uint32_t (&off)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = wave_row0 + 8 * i + (lane >> 3);
    const int chunk = (lane & 7) ^ (r & 7);
    const int gr = min(row_base + r, rows_valid - 1);
    off[i] = (uint32_t)(((int64_t)gr * ld + 8 * chunk) * 2);
  }
}

__device__ __forceinline__ void load_rows_lds(const uint16_t* __restrict__ g, int k0, const uint32_t (&off)[4],
                                              uint16_t* lds_stage, int wave_row0) {
  const char* base = reinterpret_cast<const char*>(g + k0);  // wave-uniform
#pragma unroll
  for (int i = 0; i < 4; ++i)
    __builtin_amdgcn_global_load_lds((const void*)(base + off[i]), (lds_void*)(lds_stage + (wave_row0 + 8 * i) * G_BK),
                                     16, 0, 0);
}

__global__ __launch_bounds__(G_THREADS) void gemm_had_kernel(const uint16_t* __restrict__ A,
                                                             const uint16_t* __restrict__ B,
                                                             uint16_t* __restrict__ y, int32_t P, int32_t Q,
                                                             int32_t K, int64_t ldy, int32_t n0,
                                                             const uint16_t* __restrict__ sign_n) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * G_STAGE];

  const int tiles_q = (Q + G_BQ - 1) / G_BQ;
  const int tiles = ((P + G_BP - 1) / G_BP) * tiles_q;
  const int per_xcd = (tiles + 7) / 8;
  const int t = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
  if (t >= tiles) return;  // whole workgroup (uniform)
  const int p_base = (t / tiles_q) * G_BP, q_base = (t % tiles_q) * G_BQ;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wp = wave & 1, wq = wave >> 1;

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  uint32_t offa[4], offb[4];
  lane_offsets(K, p_base, P, 32 * wave, lane, offa);
  lane_offsets(K, q_base, Q, 32 * wave, lane, offb);
  auto issue_loads = [&](int stage, int k0) {
    uint16_t* st = smem + stage * G_STAGE;
    load_rows_lds(A, k0, offa, st, 32 * wave);
    load_rows_lds(B, k0, offb, st + G_BP * G_BK, 32 * wave);
  };

  const int nk = K / G_BK;
  const int lrow = lane & 31, lhalf = lane >> 5;
  // fragments of one k16 sub-step: 4 A tiles and 2 B tiles, two register sets
  f16x8 af[2][4], bf[2][2];
  auto read_frags = [&](int stage, int s, int buf) {
    const uint16_t* As = smem + stage * G_STAGE;
    const uint16_t* Bs = As + G_BP * G_BK;
    const int ch = 2 * s + lhalf;
#pragma unroll
    for (int i = 0; i < 4; ++i) af[buf][i] = *reinterpret_cast<const f16x8*>(&As[swz(128 * wp + 32 * i + lrow, ch)]);
#pragma unroll
    for (int j = 0; j < 2; ++j) bf[buf][j] = *reinterpret_cast<const f16x8*>(&Bs[swz(64 * wq + 32 * j + lrow, ch)]);
  };
  auto mfmas = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[buf][i], bf[buf][j], acc[i][j], 0, 0, 0);
  };

  // Schedule per k step kb (stage buffer b = kb & 1):
  //   sub-steps 0..2: read the next sub-step's fragments, then MFMAs;
  //   sub-step 3: its fragments are in registers; wait for this wave's loads of
  //   stage kb+1, barrier (every wave is done reading buffer b and stage kb+1
  //   has landed), issue the loads of stage kb+2 into buffer b, read sub-step 0
  //   of stage kb+1, and only then run sub-step 3's MFMAs, which cover the
  //   barrier and the fragment-read latency.
  issue_loads(0, 0);
  if (nk > 1) issue_loads(1, G_BK);
  if (nk > 1)
    asm volatile("s_waitcnt vmcnt(8)" ::: "memory");  // stage 0 (8 loads per wave per stage)
  else
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  read_frags(0, 0, 0);
  for (int kb = 0; kb < nk; ++kb) {
    const int b = kb & 1;
    read_frags(b, 1, 1);
    mfmas(0);
    __builtin_amdgcn_sched_barrier(0);
    read_frags(b, 2, 0);
    mfmas(1);
    __builtin_amdgcn_sched_barrier(0);
    read_frags(b, 3, 1);
    mfmas(0);
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (kb + 2 < nk) issue_loads(b, (kb + 2) * G_BK);
    if (kb + 1 < nk) read_frags(b ^ 1, 0, 0);
    mfmas(1);
    __builtin_amdgcn_sched_barrier(0);
  }

  // Epilogue. acc[i][j][r] holds D[p][q] with (inside the wave's 128-row
  // rotation block) p = 32 i + 8 (r >> 2) + 4 lhalf + (r & 3), q = 32 j + lrow.
  // Index bits of p: 0,1 <- r&3; 2 <- lhalf; 3,4 <- r>>2; 5,6 <- i.
#pragma unroll
  for (int j = 0; j < 2; ++j) {
#pragma unroll
    for (int h = 1; h <= 8; h <<= 1) {  // register bits r&1, r&2, r&4, r&8
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if ((r & h) == 0) {
            const float a = acc[i][j][r], b = acc[i][j][r + h];
            acc[i][j][r] = a + b;
            acc[i][j][r + h] = a - b;
          }
    }
#pragma unroll
    for (int h = 1; h <= 2; h <<= 1) {  // register bits of i
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if ((i & h) == 0)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float a = acc[i][j][r], b = acc[i + h][j][r];
            acc[i][j][r] = a + b;
            acc[i + h][j][r] = a - b;
          }
    }
    const float s = lhalf ? -1.f : 1.f;  // lane bit: partner 32 lanes away
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float partner = __shfl_xor(acc[i][j][r], 32);
        acc[i][j][r] = __builtin_fmaf(s, acc[i][j][r], partner);
      }
  }

  const int pw = p_base + 128 * wp;  // first output column of this wave's block
  if (pw < P) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int q = q_base + 64 * wq + 32 * j + lrow;
      if (q < Q) {
        uint16_t* yrow = y + (int64_t)q * ldy + n0 + pw;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int p = 32 * i + 8 * g + 4 * lhalf;
            u32x2 o;
            o[0] = pack_f16x2(acc[i][j][4 * g] * EXL3_INV_SQRT128, acc[i][j][4 * g + 1] * EXL3_INV_SQRT128);
            o[1] = pack_f16x2(acc[i][j][4 * g + 2] * EXL3_INV_SQRT128, acc[i][j][4 * g + 3] * EXL3_INV_SQRT128);
            if (sign_n) o ^= (*reinterpret_cast<const u32x2*>(sign_n + n0 + pw + p) & 0x80008000u);
            *reinterpret_cast<u32x2*>(yrow + p) = o;
          }
      }
    }
  }
}

hipError_t launch_gemm_had(const uint16_t* A, const uint16_t* B, uint16_t* y, int32_t P, int32_t Q, int32_t K,
                           int64_t ldy, int32_t n0, const uint16_t* sign_n, hipStream_t stream) {
  const int tiles = ((P + G_BP - 1) / G_BP) * ((Q + G_BQ - 1) / G_BQ);
  const int grid = 8 * ((tiles + 7) / 8);
  gemm_had_kernel<<<grid, G_THREADS, 0, stream>>>(A, B, y, P, Q, K, ldy, n0, sign_n);
  return hipGetLastError();
}

}  // namespace exl3
