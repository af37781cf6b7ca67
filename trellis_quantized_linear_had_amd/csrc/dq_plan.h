// Work decomposition of the dequant-in-GEMM (host and device share it).
#pragma once

#include <stdint.h>

namespace exl3 {

// Units are 256 columns x one pass of 32 nqb rows, numbered pass-major. The
// first `full` units run over all of K with the output stage in the kernel;
// the `tail` units after them are split along K into tail_ks pieces of
// ksub_per_piece 16-wide k steps (the last may be short), summed by a fixup.
struct DqPlan {
  int32_t nqb;             // 32-row fragments per pass and wave (1, 2, 4 or 8)
  int32_t passes;          // passes of 32 nqb rows over M
  int32_t pblocks;         // 256-column blocks over N
  int32_t full;            // units computed whole
  int32_t tail;            // units split along K
  int32_t tail_ks;         // pieces per tail unit
  int32_t ksub_per_piece;  // 16-wide k steps per piece
};

}  // namespace exl3
