// Optional per-launch timing marks. A caller that wants the duration of one
// kernel inside a multi-kernel call passes a Marks record it owns (events it
// created, a capacity and a use count); every launch of the record's kind then
// records one event pair on its own stream. The product entry points pass no
// record, so nothing is recorded and no state is kept between calls.
#pragma once

#include <hip/hip_runtime.h>

namespace exl3 {

enum MarkKind { kMarkDecode = 0, kMarkGemm = 1, kMarkLogits = 2, kMarkReconstruct = 3, kMarkKinds = 4 };

struct Marks {
  int kind;           // which launches are marked
  int capacity;       // event pairs available
  int used;           // event pairs recorded so far
  hipEvent_t* start;  // capacity events each, created by the caller
  hipEvent_t* stop;
  int variant;        // kernel choice of exl3_linear: 0 = the library's own, else a KernelVariant
};

// Kernel sequences of exl3_linear a measurement caller may force, to time
// them against each other at the same shape.
enum KernelVariant {
  kVariantAuto = 0,
  kVariantFused = 1,
  kVariantReconstructGemm = 2,
  kVariantDequantGemm = 3,
  kVariantDequantGemmWhole = 4,  // the dequant-GEMM with every unit over all of K (no split tail)
  kVariantDequantGemm8 = 5,      // the eight-wave dequant-GEMM (256-row passes, Xr staged in LDS)
  kVariantDequantGemm8Whole = 6,  // the eight-wave dequant-GEMM with every unit over all of K
  kVariantLast = 6
};

inline hipError_t mark_begin(Marks* m, int kind, hipStream_t s) {
  if (!m || m->kind != kind || m->used >= m->capacity) return hipSuccess;
  return hipEventRecord(m->start[m->used], s);
}

inline hipError_t mark_end(Marks* m, int kind, hipStream_t s) {
  if (!m || m->kind != kind || m->used >= m->capacity) return hipSuccess;
  const hipError_t e = hipEventRecord(m->stop[m->used], s);
  if (e == hipSuccess) ++m->used;
  return e;
}

}  // namespace exl3
