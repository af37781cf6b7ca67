// Measured ceilings for the roofline fractions (not on the hot path): the
// rate of random 16-bit reads from a 128 KiB LDS table (the decode and
// reconstruct kernels' codebook gathers), a loop of independent
// v_mfma_f32_32x32x16_f16 (the prefill GEMM's instruction), and HBM streams
// (read only, write only) with 16-byte accesses. Each compute probe runs one
// workgroup per CU and records, per workgroup, the shader-clock counter
// (s_memtime) and the 100 MHz real-time counter (s_memrealtime) around its
// loop, so the host can derive the clock the loop ran at.
#include "common.h"

namespace exl3 {

#define PROBE_CUS 256

// Random u16 gathers: every lane reads 16 entries at independent uniform
// addresses (a murmur3-style finalizer of its thread index and the read
// number), issued before their sum is formed, as in the decode kernel. Each
// iteration XORs every address with one constant, which permutes the banks
// alike for all lanes (a read instruction keeps its bank-conflict pattern)
// and keeps the reads inside the loop. (Per-lane linear congruential
// sequences started at an arithmetic progression of seeds, as an earlier
// version used, stay an arithmetic progression across the lanes of one
// instruction: evenly spaced addresses with few bank conflicts, 11.66 reads
// per CU per clock against 9.06 for independent random ones.)
__global__ __launch_bounds__(1024) void probe_lds_gather_kernel(int64_t iters, uint32_t* __restrict__ sink,
                                                                uint64_t* __restrict__ clocks) {
  __shared__ uint16_t tab[65536];
  for (int i = threadIdx.x; i < 65536; i += 1024) tab[i] = (uint16_t)(i * 40503u);
  __syncthreads();
  uint32_t a[16];  // byte offsets of 16-bit entries
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    uint32_t h = (blockIdx.x * 1024u + threadIdx.x) * 16u + (uint32_t)j + 0x9E3779B9u;
    h ^= h >> 16;
    h *= 0x85EBCA6Bu;
    h ^= h >> 13;
    h *= 0xC2B2AE35u;
    h ^= h >> 16;
    a[j] = (h >> 16) << 1;
  }
  const uint64_t t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  uint32_t acc = 0;
  for (int64_t it = 0; it < iters; ++it) {
    const uint32_t c = ((uint32_t)it * 40503u & 0xFFFFu) << 1;  // even, below 2^17: stays inside the table
    uint32_t g[16];
#pragma unroll
    for (int j = 0; j < 16; ++j)
      g[j] = *reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(tab) + (a[j] ^ c));
#pragma unroll
    for (int j = 0; j < 16; ++j) acc += g[j];
  }
  __syncthreads();
  const uint64_t t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  sink[blockIdx.x * 1024 + threadIdx.x] = acc;
  if (threadIdx.x == 0) {
    clocks[4 * blockIdx.x + 0] = t0;
    clocks[4 * blockIdx.x + 1] = t1;
    clocks[4 * blockIdx.x + 2] = r0;
    clocks[4 * blockIdx.x + 3] = r1;
  }
}

// Independent MFMAs: 8 waves (two per SIMD), 8 accumulators per wave. The
// operands are fp16 values of mixed sign and magnitude whose low mantissa
// bits change every iteration (two VALU ops per 8 MFMAs), so the multipliers
// switch as they do on real data.
__global__ __launch_bounds__(512) void probe_mfma_kernel(int64_t iters, float* __restrict__ sink,
                                                         uint64_t* __restrict__ clocks) {
  const int lane = threadIdx.x & 63;
  u32x4 ab, bb;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // exponents 2^-1 .. 2^-4, both signs, lane-dependent mantissas
    const uint32_t h = (uint32_t)(lane * 0x9E3779B9u) ^ (uint32_t)(j * 0x85EBCA6Bu) ^ (blockIdx.x * 0x27D4EB2Fu);
    ab[j] = (h & 0x83FF83FFu) | 0x34003800u;
    bb[j] = ((h >> 7) & 0x83FF83FFu) | 0x38003400u;
  }
  f32x16 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
  __syncthreads();
  const uint64_t t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int64_t it = 0; it < iters; ++it) {
    const uint32_t flip = ((uint32_t)it * 0x00050003u) & 0x007F007Fu;  // low mantissa bits only
    ab ^= flip;
    bb ^= flip << 1;
    const f16x8 a = __builtin_bit_cast(f16x8, ab), b = __builtin_bit_cast(f16x8, bb);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[i], 0, 0, 0);
  }
  __syncthreads();
  const uint64_t t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[i][r];
  sink[blockIdx.x * 512 + threadIdx.x] = s;
  if (threadIdx.x == 0) {
    clocks[4 * blockIdx.x + 0] = t0;
    clocks[4 * blockIdx.x + 1] = t1;
    clocks[4 * blockIdx.x + 2] = r0;
    clocks[4 * blockIdx.x + 3] = r1;
  }
}

// HBM streams over n16 16-byte chunks, grid-stride: READ xors every chunk
// into one value per thread (stored to sink); WRITE stores a pattern.
template <bool READ>
__global__ __launch_bounds__(256) void probe_stream_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                           int64_t n16, uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (READ) {
    u32x4 acc = {0, 0, 0, 0};
    for (; i + 3 * stride < n16; i += 4 * stride) {
      const u32x4 v0 = src[i], v1 = src[i + stride], v2 = src[i + 2 * stride], v3 = src[i + 3 * stride];
      acc ^= v0 ^ v1 ^ v2 ^ v3;
    }
    for (; i < n16; i += stride) acc ^= src[i];
    sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  } else {
    const u32x4 v = {(uint32_t)i, 0x3C003C00u, 0u, 0xFFFFFFFFu};
    for (; i < n16; i += stride) dst[i] = v;
  }
}

// Row-pattern read: the buffer as rows of PROBE_ROW_BYTES; a wave owns 128
// rows and walks them in 128-byte column chunks, each 16-byte load
// instruction reading whole 128-byte lines of 8 rows (lane l: row 8 i + l / 8,
// piece l % 8), non-temporal: the weight stream of the padded-logits GEMM.
// The next chunk's 16 loads are issued before the current chunk is consumed.
#define PROBE_ROW_BYTES 10240
__device__ __forceinline__ void probe_rows_chunk(const char* const (&rp)[16], int kc, u32x4 (&v)[16]) {
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(rp[i] + kc));
}

__global__ __launch_bounds__(256) void probe_rows_kernel(const char* __restrict__ src, int64_t waves,
                                                         uint32_t* __restrict__ sink) {
  const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= waves) return;
  const int lane = threadIdx.x & 63;
  const char* rp[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) rp[i] = src + (w * 128 + 8 * i + (lane >> 3)) * PROBE_ROW_BYTES + 16 * (lane & 7);
  u32x4 acc = {0, 0, 0, 0}, v0[16], v1[16];
  probe_rows_chunk(rp, 0, v0);
  for (int kc = 0; kc < PROBE_ROW_BYTES; kc += 256) {
    probe_rows_chunk(rp, kc + 128, v1);
#pragma unroll
    for (int i = 0; i < 16; ++i) acc ^= v0[i];
    if (kc + 256 < PROBE_ROW_BYTES) probe_rows_chunk(rp, kc + 256, v0);
#pragma unroll
    for (int i = 0; i < 16; ++i) acc ^= v1[i];
  }
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

hipError_t launch_probe_lds_gather(int64_t iters, uint32_t* sink, uint64_t* clocks, hipStream_t stream) {
  probe_lds_gather_kernel<<<PROBE_CUS, 1024, 0, stream>>>(iters, sink, clocks);
  return hipGetLastError();
}

hipError_t launch_probe_mfma(int64_t iters, float* sink, uint64_t* clocks, hipStream_t stream) {
  probe_mfma_kernel<<<PROBE_CUS, 512, 0, stream>>>(iters, sink, clocks);
  return hipGetLastError();
}

hipError_t launch_probe_stream(int32_t write, const void* src, void* dst, int64_t bytes, uint32_t* sink,
                               hipStream_t stream) {
  const int64_t n16 = bytes / 16;
  if (write == 2) {  // row-pattern read of the whole 128-row groups that fit
    const int64_t waves = bytes / PROBE_ROW_BYTES / 128;
    if (waves == 0) return hipSuccess;
    probe_rows_kernel<<<(unsigned)((waves + 3) / 4), 256, 0, stream>>>((const char*)src, waves, sink);
    return hipGetLastError();
  }
  if (write)
    probe_stream_kernel<false><<<PROBE_CUS * 32, 256, 0, stream>>>(nullptr, (u32x4*)dst, n16, sink);
  else
    probe_stream_kernel<true><<<PROBE_CUS * 32, 256, 0, stream>>>((const u32x4*)src, nullptr, n16, sink);
  return hipGetLastError();
}

}  // namespace exl3
