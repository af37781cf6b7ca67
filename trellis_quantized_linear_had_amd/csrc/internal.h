// Entry points of libexl3 below its C ABI, for callers built against the
// library that also pass timing marks (marks.h). The exported C functions
// are these with no marks.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "exl3.h"

namespace exl3 {

struct Marks;

// exl3_linear with optional marks (kMarkDecode, kMarkReconstruct, kMarkGemm).
int linear_entry(const exl3_layer* L, const uint16_t* x, int64_t M, uint16_t* y, void* scratch, size_t scratch_bytes,
                 int32_t prefill_min_m, hipStream_t stream, Marks* marks);

// Scratch of exl3_linear with its kernel sequence forced (marks.h variants).
size_t linear_variant_scratch_bytes(int32_t K, int32_t N, int64_t M, int32_t prefill_min_m, int variant);

// exl3_head_logits_argmax with optional marks (kMarkDecode, kMarkReconstruct,
// kMarkGemm).
int head_entry(const exl3_layer* L, const uint16_t* x, int64_t M, int64_t n_valid, uint16_t* logits,
               int64_t ld_logits, int64_t* argmax, void* scratch, size_t scratch_bytes, int32_t prefill_min_m,
               hipStream_t stream, Marks* marks);

// logits_pad_mask_argmax with optional marks (kMarkLogits).
int logits_entry(const uint16_t* x, int64_t M, int32_t K, const uint16_t* w, int64_t w_rows, int64_t n_valid,
                 uint16_t* logits, int64_t ld_logits, int64_t* argmax, void* scratch, size_t scratch_bytes,
                 hipStream_t stream, Marks* marks);

}  // namespace exl3
