/*
 * measure.h -- C ABI of libexl3_measure.so, the measurement companion of
 * libexl3.so: per-kernel timing of the library's calls with caller-owned HIP
 * events, and probes of the chip's ceilings (LDS random gathers, an fp16 MFMA
 * loop, HBM read and write streams). Benchmarks and their tests load it; the
 * product library has no timing state and no probes.
 *
 * All pointers are device pointers unless stated; `stream` is a hipStream_t.
 * Functions return the libexl3 status codes (EXL3_OK = 0; exl3.h).
 */
#ifndef EXL3_MEASURE_H
#define EXL3_MEASURE_H

#include <stddef.h>
#include <stdint.h>

#include "exl3.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Kinds of marked launches. */
#define EXL3M_DECODE 0      /* the decode GEMM of exl3_linear's fused path */
#define EXL3M_GEMM 1        /* the full-tile launch of the prefill GEMM, one per column slice */
#define EXL3M_LOGITS 2      /* the logits GEMM, one per 16-row group */
#define EXL3M_RECONSTRUCT 3 /* the prefill path's reconstruct of one column slice */

/* Creates n timing events (host handles written to events[0..n)). */
int exl3m_events_create(int n, void **events);
/* Destroys n events created by exl3m_events_create. */
int exl3m_events_destroy(int n, void **events);
/* Waits for event b, then *ms = time from a to b in milliseconds. */
int exl3m_elapsed_ms(void *a, void *b, float *ms);

/* Kernel sequences of exl3_linear that a measurement may force. */
#define EXL3M_VARIANT_AUTO 0         /* the library's own choice */
#define EXL3M_VARIANT_FUSED 1        /* decode-GEMM + output stage */
#define EXL3M_VARIANT_RECON_GEMM 2   /* reconstruct + MFMA GEMM */
#define EXL3M_VARIANT_DEQUANT_GEMM 3 /* dequant-in-GEMM (its own output stage; a K-split tail and fixup) */
#define EXL3M_VARIANT_DEQUANT_WHOLE 4 /* the same with every unit over all of K */

/* exl3_linear, with one event pair recorded on `stream` around every launch
 * of `kind` (start[i] before, stop[i] after), at most `capacity` pairs;
 * *used = the pairs recorded. `variant` forces a kernel sequence (the
 * dequant-GEMM marks as EXL3M_DECODE); EXL3M_VARIANT_AUTO is exl3_linear's
 * own dispatch. */
int exl3m_linear_marked(const exl3_layer *layer, const uint16_t *x, int64_t M, uint16_t *y, void *scratch,
                        size_t scratch_bytes, int32_t prefill_min_m, void *stream, int kind, int capacity,
                        void **start, void **stop, int *used, int variant);

/* Scratch bytes exl3m_linear_marked needs with this variant (0 for invalid
 * shapes); EXL3M_VARIANT_AUTO gives exl3_linear_scratch_bytes. */
size_t exl3m_linear_scratch_bytes(int32_t K, int32_t N, int64_t M, int32_t prefill_min_m, int variant);

/* exl3_head_logits_argmax with marks, as exl3m_linear_marked. */
int exl3m_head_marked(const exl3_layer *layer, const uint16_t *x, int64_t M, int64_t n_valid, uint16_t *logits,
                      int64_t ld_logits, int64_t *argmax, void *scratch, size_t scratch_bytes, int32_t prefill_min_m,
                      void *stream, int kind, int capacity, void **start, void **stop, int *used);

/* logits_pad_mask_argmax with marks, as exl3m_linear_marked. */
int exl3m_logits_marked(const uint16_t *x, int64_t M, int32_t K, const uint16_t *w, int64_t w_rows, int64_t n_valid,
                        uint16_t *logits, int64_t ld_logits, int64_t *argmax, void *scratch, size_t scratch_bytes,
                        void *stream, int kind, int capacity, void **start, void **stop, int *used);

/* Probes. Each launches EXL3M_PROBE_WORKGROUPS workgroups on `stream` and
 * returns at once.
 *   exl3m_probe_lds_gather: every lane issues `iters` x 16 random 16-bit reads
 *     from a 128 KiB LDS table at addresses independent across lanes (the
 *     codebook gathers of the trellis kernels, whose states come from a
 *     random bitstream);
 *   exl3m_probe_mfma: 8 waves per workgroup each issue `iters` x 8 independent
 *     v_mfma_f32_32x32x16_f16 (32768 FLOP each);
 *   exl3m_probe_stream: write = 0 reads `bytes` of src in 16-byte accesses,
 *     1 fills `bytes` of dst, 2 reads src as rows of 10240 bytes in the
 *     padded-logits GEMM's pattern (each 16-byte load instruction reads a
 *     whole 128-byte line of each of 8 rows, non-temporal; whole groups of
 *     128 rows only, so
 *     floor(bytes / 1310720) * 1310720 bytes); bytes a multiple of 16.
 * sink: device buffer of EXL3M_PROBE_SINK_BYTES that keeps the results live.
 * clocks (compute probes): device buffer of 4 x EXL3M_PROBE_WORKGROUPS uint64:
 * per workgroup the shader-clock counter (s_memtime) before and after its
 * loop, then the 100 MHz real-time counter (s_memrealtime) before and after.
 * EXL3_EINVAL for NULL or misaligned pointers, negative sizes, an unknown
 * stream mode or a byte count that is not a multiple of 16. */
#define EXL3M_PROBE_WORKGROUPS 256
#define EXL3M_PROBE_SINK_BYTES (256 * 32 * 256 * 4)
int exl3m_probe_lds_gather(int64_t iters, uint32_t *sink, uint64_t *clocks, void *stream);
int exl3m_probe_mfma(int64_t iters, float *sink, uint64_t *clocks, void *stream);
int exl3m_probe_stream(int32_t write, const void *src, void *dst, int64_t bytes, uint32_t *sink, void *stream);

/* Text for the most recent failure of a measurement call on this thread
 * (or libexl3's message for a failing library call). */
const char *exl3m_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* EXL3_MEASURE_H */
