// libexl3_measure.so: per-kernel timing marks over libexl3's calls and the
// ceiling probes (measure.h). Links against libexl3.so; holds no state of its
// own between calls.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>

#include "internal.h"
#include "marks.h"
#include "measure.h"

namespace exl3 {
hipError_t launch_probe_lds_gather(int64_t iters, uint32_t* sink, uint64_t* clocks, hipStream_t stream);
hipError_t launch_probe_mfma(int64_t iters, float* sink, uint64_t* clocks, hipStream_t stream);
hipError_t launch_probe_stream(int32_t write, const void* src, void* dst, int64_t bytes, uint32_t* sink,
                               hipStream_t stream);
}  // namespace exl3

namespace {

thread_local char m_msg[256];
thread_local bool m_own = false;  // the last failure is this library's, not libexl3's

int mfail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int mfail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(m_msg, sizeof(m_msg), fmt, ap);
  va_end(ap);
  m_own = true;
  return status;
}

int mhip(hipError_t e, const char* where) {
  return e == hipSuccess ? EXL3_OK : mfail(EXL3_EHIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int make_marks(exl3::Marks& m, int kind, int capacity, void** start, void** stop, int* used, int variant = 0) {
  if (kind < 0 || kind >= exl3::kMarkKinds) return mfail(EXL3_EINVAL, "mark kind %d is not 0..3", kind);
  if (variant < 0 || variant > exl3::kVariantLast) return mfail(EXL3_EINVAL, "variant %d is not 0..%d", variant, (int)exl3::kVariantLast);
  if (capacity < 0 || (capacity > 0 && (!start || !stop)) || !used)
    return mfail(EXL3_EINVAL, "bad event arrays (capacity %d)", capacity);
  m = exl3::Marks{kind, capacity, 0, reinterpret_cast<hipEvent_t*>(start), reinterpret_cast<hipEvent_t*>(stop),
                  variant};
  return EXL3_OK;
}

}  // namespace

extern "C" {

int exl3m_events_create(int n, void** events) {
  m_own = false;
  if (n < 0 || (n > 0 && !events)) return mfail(EXL3_EINVAL, "n = %d or events NULL", n);
  for (int i = 0; i < n; ++i) {
    hipEvent_t e = nullptr;
    const int st = mhip(hipEventCreate(&e), "hipEventCreate");
    if (st) {
      for (int j = 0; j < i; ++j) (void)hipEventDestroy(reinterpret_cast<hipEvent_t>(events[j]));
      return st;
    }
    events[i] = e;
  }
  return EXL3_OK;
}

int exl3m_events_destroy(int n, void** events) {
  m_own = false;
  if (n < 0 || (n > 0 && !events)) return mfail(EXL3_EINVAL, "n = %d or events NULL", n);
  int st = EXL3_OK;
  for (int i = 0; i < n; ++i) {
    const int s = mhip(hipEventDestroy(reinterpret_cast<hipEvent_t>(events[i])), "hipEventDestroy");
    if (!st) st = s;
  }
  return st;
}

int exl3m_elapsed_ms(void* a, void* b, float* ms) {
  m_own = false;
  if (!a || !b || !ms) return mfail(EXL3_EINVAL, "NULL event or output");
  int st = mhip(hipEventSynchronize(reinterpret_cast<hipEvent_t>(b)), "hipEventSynchronize");
  if (st) return st;
  return mhip(hipEventElapsedTime(ms, reinterpret_cast<hipEvent_t>(a), reinterpret_cast<hipEvent_t>(b)),
              "hipEventElapsedTime");
}

int exl3m_linear_marked(const exl3_layer* layer, const uint16_t* x, int64_t M, uint16_t* y, void* scratch,
                        size_t scratch_bytes, int32_t prefill_min_m, void* stream, int kind, int capacity,
                        void** start, void** stop, int* used, int variant) {
  m_own = false;
  exl3::Marks m;
  int st = make_marks(m, kind, capacity, start, stop, used, variant);
  if (st) return st;
  st = exl3::linear_entry(layer, x, M, y, scratch, scratch_bytes, prefill_min_m, (hipStream_t)stream, &m);
  *used = m.used;
  return st;
}

size_t exl3m_linear_scratch_bytes(int32_t K, int32_t N, int64_t M, int32_t prefill_min_m, int variant) {
  if (variant < 0 || variant > exl3::kVariantLast) return 0;
  return exl3::linear_variant_scratch_bytes(K, N, M, prefill_min_m, variant);
}

int exl3m_head_marked(const exl3_layer* layer, const uint16_t* x, int64_t M, int64_t n_valid, uint16_t* logits,
                      int64_t ld_logits, int64_t* argmax, void* scratch, size_t scratch_bytes, int32_t prefill_min_m,
                      void* stream, int kind, int capacity, void** start, void** stop, int* used) {
  m_own = false;
  exl3::Marks m;
  int st = make_marks(m, kind, capacity, start, stop, used);
  if (st) return st;
  st = exl3::head_entry(layer, x, M, n_valid, logits, ld_logits, argmax, scratch, scratch_bytes, prefill_min_m,
                        (hipStream_t)stream, &m);
  *used = m.used;
  return st;
}

int exl3m_logits_marked(const uint16_t* x, int64_t M, int32_t K, const uint16_t* w, int64_t w_rows, int64_t n_valid,
                        uint16_t* logits, int64_t ld_logits, int64_t* argmax, void* scratch, size_t scratch_bytes,
                        void* stream, int kind, int capacity, void** start, void** stop, int* used) {
  m_own = false;
  exl3::Marks m;
  int st = make_marks(m, kind, capacity, start, stop, used);
  if (st) return st;
  st = exl3::logits_entry(x, M, K, w, w_rows, n_valid, logits, ld_logits, argmax, scratch, scratch_bytes,
                          (hipStream_t)stream, &m);
  *used = m.used;
  return st;
}

int exl3m_probe_lds_gather(int64_t iters, uint32_t* sink, uint64_t* clocks, void* stream) {
  m_own = false;
  if (iters < 0) return mfail(EXL3_EINVAL, "iters = %lld is negative", (long long)iters);
  if (!sink || !clocks || !aligned16(sink) || !aligned16(clocks))
    return mfail(EXL3_EINVAL, "sink or clocks NULL or misaligned");
  return mhip(exl3::launch_probe_lds_gather(iters, sink, clocks, (hipStream_t)stream), "lds gather probe");
}

int exl3m_probe_mfma(int64_t iters, float* sink, uint64_t* clocks, void* stream) {
  m_own = false;
  if (iters < 0) return mfail(EXL3_EINVAL, "iters = %lld is negative", (long long)iters);
  if (!sink || !clocks || !aligned16(sink) || !aligned16(clocks))
    return mfail(EXL3_EINVAL, "sink or clocks NULL or misaligned");
  return mhip(exl3::launch_probe_mfma(iters, sink, clocks, (hipStream_t)stream), "mfma probe");
}

int exl3m_probe_stream(int32_t write, const void* src, void* dst, int64_t bytes, uint32_t* sink, void* stream) {
  m_own = false;
  if (bytes < 0 || bytes % 16)
    return mfail(EXL3_EINVAL, "bytes = %lld must be a non-negative multiple of 16", (long long)bytes);
  if (write < 0 || write > 2) return mfail(EXL3_EINVAL, "stream mode %d is not 0, 1 or 2", write);
  const void* buf = write == 1 ? dst : src;
  if (!buf || !aligned16(buf) || !sink || !aligned16(sink))
    return mfail(EXL3_EINVAL, "stream buffer or sink NULL or misaligned");
  if (bytes == 0) return EXL3_OK;
  return mhip(exl3::launch_probe_stream(write, src, dst, bytes, sink, (hipStream_t)stream), "stream probe");
}

const char* exl3m_strerror(int status) {
  if (status == EXL3_OK) return "ok";
  return m_own ? m_msg : exl3_strerror(status);
}

}  // extern "C"
