// Work decomposition of the fused decode-GEMM (host and device share it).
#pragma once

#include <stdint.h>

// Most n-tiles (16 columns each) one workgroup keeps accumulators and an LDS
// reduction slot for.
#define DEC_NT_MAX 24

// LDS the decode kernel keeps beside the 128 KiB codebook for the rotated
// activation slice (rows < M, the workgroup's k range, fp16).
#define DEC_XS_BYTES 32768

namespace exl3 {

struct DecodePlan {
  int32_t ks_count;       // workgroups along K
  int32_t ns_count;       // workgroups along N
  int32_t ksteps_per_wg;  // 32-wide k-steps per workgroup (last may be short)
  int32_t ntiles_per_wg;  // 16-wide n-tiles per workgroup (last may be short), <= DEC_NT_MAX
  int32_t wn;             // waves along N inside a workgroup
  int32_t wk;             // waves along K inside a workgroup (wn * wk = 16)
  int32_t nt_wave;        // compiled n-tiles per wave (>= the largest wave share)
  int32_t x_in_lds;       // 1: each workgroup rotates its own x slice into LDS
                          // (M <= 16, slice <= DEC_XS_BYTES); 0: x is rotated
                          // by a separate pass into scratch
  int32_t groups;         // 16-row groups per pass sharing each decoded tile (1, 2, 4)
};

// Per-wave n-tile counts the decode kernel is compiled for (16 waves of at
// most 128 VGPRs: accumulators and two code-word sets grow with the count;
// 12 no longer fits without spilling).
static const int32_t kDecodeNtInstances[] = {1, 2, 3, 4, 5, 6, 8, 9, 10};
// ... and with 2 or 4 row groups per pass (accumulators grow with the groups)
static const int32_t kDecodeNtInstancesG2[] = {1, 2, 3, 4, 5};
static const int32_t kDecodeNtInstancesG4[] = {1, 2, 3};
// ... and at widths other than 4 bits (up to three code words per tile and
// lane): one, two or four row groups per pass
static const int32_t kDecodeNtInstancesOther[] = {2, 3, 4, 5, 6};
static const int32_t kDecodeNtInstancesOtherG2[] = {2, 3, 4, 5};
static const int32_t kDecodeNtInstancesOtherG4[] = {1, 2};

}  // namespace exl3
