// Work decomposition of the dequant-in-GEMM (host and device share it).
#pragma once

#include <stdint.h>

namespace exl3 {

// Units are 256 columns x one pass of 32 nqb rows, numbered pass-major. The
// first `full` units run over all of K with the output stage in the kernel;
// the `tail` units after them are split along K, summed by a fixup: either
// into tail_ks pieces of ksub_per_piece 16-wide k steps per unit (the last
// may be short), or (sk_steps > 0, the eight-wave kernel) stream-K: the tail
// units' 32-wide k steps, unit-major, dealt in runs of sk_steps to sk_wgs
// workgroups, each run touching at most two units (sk_steps <= K / 32) and
// leaving one partial per unit it touches (slot run + tail unit: sk_wgs +
// tail - 1 slots).
struct DqPlan {
  int32_t nqb;             // 32-row fragments per pass and wave (1, 2, 4 or 8)
  int32_t passes;          // passes of 32 nqb rows over M
  int32_t pblocks;         // 256-column blocks over N
  int32_t full;            // units computed whole
  int32_t tail;            // units split along K
  int32_t tail_ks;         // pieces per tail unit
  int32_t ksub_per_piece;  // 16-wide k steps per piece
  int32_t sk_steps;        // stream-K: 32-wide k steps per workgroup (0: pieces per unit)
  int32_t sk_wgs;          // stream-K: workgroups
};

}  // namespace exl3
