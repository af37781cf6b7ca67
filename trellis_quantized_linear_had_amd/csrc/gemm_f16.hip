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
// Tiling: 256 (p) x 128 (q) per workgroup, 64-wide k steps staged through LDS
// (double-buffered, 16-byte chunks XOR-swizzled by row so the fragment reads
// are bank-conflict free); 4 waves as 2 x 2, each 128 (p) x 64 (q) = 4 x 2
// v_mfma_f32_32x32x16_f16 tiles.
#include "common.h"

namespace exl3 {

#define G_BP 256
#define G_BQ 128
#define G_BK 64
#define G_THREADS 256

__device__ __forceinline__ int swz(int row, int chunk) { return row * G_BK + ((chunk ^ (row & 7)) << 3); }

__global__ __launch_bounds__(G_THREADS) void gemm_had_kernel(const uint16_t* __restrict__ A,
                                                             const uint16_t* __restrict__ B,
                                                             uint16_t* __restrict__ y, int32_t P, int32_t Q,
                                                             int32_t K, int64_t ldy, int32_t n0,
                                                             const uint16_t* __restrict__ sign_n) {
  __shared__ uint16_t As[2][G_BP * G_BK];
  __shared__ uint16_t Bs[2][G_BQ * G_BK];

  const int nQ = (Q + G_BQ - 1) / G_BQ;
  const int pt = blockIdx.x / nQ, qt = blockIdx.x % nQ;
  const int p_base = pt * G_BP, q_base = qt * G_BQ;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wp = wave & 1, wq = wave >> 1;

  // global -> register staging: A 2048 chunks of 16 B (8 per thread), B 1024 (4 per thread)
  u32x4 ra[8], rb[4];
  auto load_global = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int id = tid + i * G_THREADS, row = id >> 3, ch = id & 7;
      const int p = p_base + row;
      ra[i] = (p < P) ? *reinterpret_cast<const u32x4*>(A + (int64_t)p * K + k0 + 8 * ch) : (u32x4){0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = tid + i * G_THREADS, row = id >> 3, ch = id & 7;
      const int q = q_base + row;
      rb[i] = (q < Q) ? *reinterpret_cast<const u32x4*>(B + (int64_t)q * K + k0 + 8 * ch) : (u32x4){0, 0, 0, 0};
    }
  };
  auto store_lds = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int id = tid + i * G_THREADS, row = id >> 3, ch = id & 7;
      *reinterpret_cast<u32x4*>(&As[buf][swz(row, ch)]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = tid + i * G_THREADS, row = id >> 3, ch = id & 7;
      *reinterpret_cast<u32x4*>(&Bs[buf][swz(row, ch)]) = rb[i];
    }
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = K / G_BK;
  load_global(0);
  store_lds(0);
  __syncthreads();
  const int lrow = lane & 31, lhalf = lane >> 5;
  for (int kb = 0; kb < nk; ++kb) {
    const int buf = kb & 1;
    if (kb + 1 < nk) load_global((kb + 1) * G_BK);
#pragma unroll
    for (int s = 0; s < G_BK / 16; ++s) {
      const int ch = 2 * s + lhalf;
      f16x8 af[4], bf[2];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const f16x8*>(&As[buf][swz(128 * wp + 32 * i + lrow, ch)]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bf[j] = *reinterpret_cast<const f16x8*>(&Bs[buf][swz(64 * wq + 32 * j + lrow, ch)]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    if (kb + 1 < nk) store_lds(buf ^ 1);
    __syncthreads();
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
  const int nP = (P + G_BP - 1) / G_BP, nQ = (Q + G_BQ - 1) / G_BQ;
  gemm_had_kernel<<<nP * nQ, G_THREADS, 0, stream>>>(A, B, y, P, Q, K, ldy, n0, sign_n);
  return hipGetLastError();
}

}  // namespace exl3
