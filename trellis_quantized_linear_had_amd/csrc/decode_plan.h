// Work decomposition of the fused decode-GEMM (host and device share it).
#pragma once

#include <stdint.h>

// Most n-tiles (16 columns each) one workgroup keeps accumulators and an LDS
// reduction slot for.
#define DEC_NT_MAX 24

namespace exl3 {

struct DecodePlan {
  int32_t ks_count;       // workgroups along K
  int32_t ns_count;       // workgroups along N
  int32_t ksteps_per_wg;  // 32-wide k-steps per workgroup (last may be short)
  int32_t ntiles_per_wg;  // 16-wide n-tiles per workgroup (last may be short), <= DEC_NT_MAX
  int32_t wn;             // waves along N inside a workgroup
  int32_t wk;             // waves along K inside a workgroup (wn * wk = 16)
  int32_t nt_wave;        // compiled n-tiles per wave (>= the largest wave share)
};

// Per-wave n-tile counts the decode kernel is compiled for (16 waves of at
// most 128 VGPRs: accumulators and two code-word sets grow with the count).
static const int32_t kDecodeNtInstances[] = {1, 2, 3, 4, 5, 6, 8, 9, 10, 12};

}  // namespace exl3
