// Host side of libexl3: argument validation (fail closed, before any launch),
// the row-count dispatch between the fused decode path and the prefill path
// (vLLM PR #316, "Change": the branch sits inside the op and is taken at call
// time; threshold 128 by default, 0 disables the prefill path), the
// <= 32768-column slice loop over one caller-owned scratch buffer, and status
// reporting. No allocation, host synchronisation, environment read or timing
// search happens in any call (vLLM PR #314, "Problem": a lazily allocated
// buffer on first call breaks graph capture).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "exl3.h"
#include "decode_plan.h"
#include "dq_plan.h"
#include "internal.h"
#include "marks.h"

namespace exl3 {
hipError_t launch_had128_frag(const uint16_t* in, uint16_t* out, int64_t M, int32_t K, const uint16_t* sign_pre,
                              bool rows16, hipStream_t stream);
hipError_t launch_had128(const uint16_t* in, uint16_t* out, int64_t rows, int64_t cols, const uint16_t* sign_pre,
                         const uint16_t* sign_post, hipStream_t stream);
hipError_t launch_reconstruct_nk(const uint32_t* codes, const uint16_t* cb, const uint16_t* scale, int32_t K,
                                 int32_t N, int32_t bits, int32_t n0, int32_t n_count, uint16_t* wt, int64_t ldw,
                                 hipStream_t stream);
hipError_t launch_reconstruct_kn(const uint32_t* codes, const uint16_t* cb, const uint16_t* scale, int32_t K,
                                 int32_t N, int32_t bits, int32_t n0, int32_t n_count, uint16_t* w, int64_t ldw,
                                 bool states, hipStream_t stream);
hipError_t launch_decode_gemm(const uint16_t* xin, const uint16_t* sign_k, const uint32_t* codes, const uint16_t* cb,
                              float* partials, int32_t K, int32_t N, int32_t ldt, int32_t M, int32_t bits,
                              const DecodePlan& plan, hipStream_t stream);
hipError_t launch_decode_finalize(const float* partials, int32_t ks_count, const uint16_t* scale,
                                  const uint16_t* sign_n, uint16_t* y, int64_t ldy, int32_t M, int32_t N,
                                  hipStream_t stream);
hipError_t launch_head_mask_argmax(uint16_t* logits, int64_t ld, int64_t M, int64_t n_valid, int64_t n_pad,
                                   int64_t* argmax, int32_t* pk, int32_t* pi, hipStream_t stream);
int64_t head_argmax_items(int64_t n_pad);
hipError_t launch_gemm_had(const uint16_t* A, const uint16_t* B, uint16_t* y, int32_t P, int32_t Q, int32_t K,
                           int64_t ldy, int32_t n0, const uint16_t* sign_n, float* partial, hipStream_t stream,
                           Marks* marks);
size_t gemm_partial_bytes(int32_t P, int32_t Q, int32_t K);
hipError_t launch_dqgemm2(const uint16_t* xf16, const uint32_t* codes, const uint16_t* cb, const uint16_t* scale,
                          const uint16_t* sign_n, uint16_t* y, int64_t ldy, float* partials, int32_t K, int32_t N,
                          int32_t ldt, int32_t M, const DqPlan& plan, hipStream_t stream);
hipError_t launch_dqgemm(const uint16_t* xf, const uint32_t* codes, const uint16_t* cb, const uint16_t* scale,
                         const uint16_t* sign_n, uint16_t* y, int64_t ldy, float* partials, int32_t K, int32_t N,
                         int32_t ldt, int32_t M, const DqPlan& plan, hipStream_t stream);
size_t dq_partial_bytes(const DqPlan& plan);
hipError_t launch_logits(const uint16_t* x, int32_t M, int32_t K, const uint16_t* w, int64_t n_valid, int64_t n_pad,
                         uint16_t* logits, int64_t ld, int64_t* argmax, int32_t* pk, int32_t* pi, uint16_t* xp,
                         hipStream_t stream, Marks* marks);
int64_t logits_items(int64_t n_pad);
size_t logits_xperm_bytes(int64_t M, int32_t K);
}  // namespace exl3

using namespace exl3;

namespace {

thread_local char g_msg[512];

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
  return status;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(EXL3_EHIP, "%s: %s", where, hipGetErrorString(e));
}

#define EXL3_TRY(call, where)                  \
  do {                                         \
    hipError_t e_ = (call);                    \
    if (e_ != hipSuccess) return hip_fail(e_, where); \
  } while (0)

// Device architecture check, cached per device (a result, not tuning state).
std::atomic<int> g_arch_ok[64];

int check_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(EXL3_EARCH, "device index %d out of range", dev);
  int st = g_arch_ok[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
    st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_arch_ok[dev].store(st, std::memory_order_relaxed);
  }
  if (st != 1) return fail(EXL3_EARCH, "device %d is not gfx950", dev);
  return EXL3_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// Shape checks shared by every call that reads packed codes.
int validate_codes_shape(const exl3_layer* L) {
  if (L->bits < 1 || L->bits > 8) return fail(EXL3_ESHAPE, "bits = %d; 1 to 8 bits per weight are supported", L->bits);
  if (L->K <= 0 || L->N <= 0 || L->K % 128 || L->N % 128)
    return fail(EXL3_ESHAPE, "K = %d and N = %d must be positive multiples of 128", L->K, L->N);
  // The kernels address the packed codes (K N bits / 8 bytes) and one fp16
  // weight slice (K x up to 32768 columns) with 32-bit byte offsets.
  if ((int64_t)L->K * L->N * L->bits / 8 > (int64_t)UINT32_MAX)
    return fail(EXL3_ESHAPE, "K = %d, N = %d, bits = %d: the packed codes exceed 4 GiB", L->K, L->N, L->bits);
  if (L->K >= 65536) return fail(EXL3_ESHAPE, "K = %d must be below 65536", L->K);
  return EXL3_OK;
}

int validate_layer(const exl3_layer* L) {
  if (!L) return fail(EXL3_EINVAL, "layer is NULL");
  if (!L->codes || !L->codebook || !L->scale) return fail(EXL3_EINVAL, "layer codes, codebook or scale is NULL");
  const int st = validate_codes_shape(L);
  if (st) return st;
  if (!aligned16(L->codes) || !aligned16(L->codebook) || !aligned16(L->scale) || !aligned16(L->sign_k) ||
      !aligned16(L->sign_n))
    return fail(EXL3_EINVAL, "layer tensors must be 16-byte aligned");
  return EXL3_OK;
}

bool use_prefill(int64_t M, int32_t prefill_min_m) { return prefill_min_m > 0 && M >= prefill_min_m; }

// Chooses (ks, ns, wn, wk, NT, G) for the decode kernel: every workgroup
// gets the same work, the grid fills at most whole rounds of 256 CUs, and the
// modelled cost (per round: the workgroup's tile-steps and the padded
// per-wave share, once per pass of G row groups, plus a round cost of about
// 4 us for the codebook load, prologue and reduction; plus the fp32 partial
// traffic and the rows of Xr that every column slice reads again) is least. The LDS gathers are the bound, so a pass
// of G groups costs about one gather pass (the extra MFMAs and A fragments add
// a few per cent per group). With x_in_lds (one group) the workgroup's k range
// is a whole number of 128-element blocks and its rotated slice of the M rows
// fits DEC_XS_BYTES.
static bool plan_decode_search(int32_t K, int32_t N, int64_t M, bool x_in_lds, int G, bool four_bits,
                               DecodePlan& best, double& best_cost) {
  const int ksteps = K / 32, ntiles = N / 16;
  const int64_t passes = (M + 16 * G - 1) / (16 * G);
  const double gfac = 1.0 + 0.05 * (G - 1);
  const int32_t* inst = nullptr;
  int ninst = 0;
  auto pick = [&](const int32_t* list, size_t bytes) {
    inst = list;
    ninst = (int)(bytes / sizeof(int32_t));
  };
  if (four_bits)
    G == 1 ? pick(kDecodeNtInstances, sizeof(kDecodeNtInstances))
    : G == 2 ? pick(kDecodeNtInstancesG2, sizeof(kDecodeNtInstancesG2))
             : pick(kDecodeNtInstancesG4, sizeof(kDecodeNtInstancesG4));
  else
    G == 1 ? pick(kDecodeNtInstancesOther, sizeof(kDecodeNtInstancesOther))
    : G == 2 ? pick(kDecodeNtInstancesOtherG2, sizeof(kDecodeNtInstancesOtherG2))
             : pick(kDecodeNtInstancesOtherG4, sizeof(kDecodeNtInstancesOtherG4));
  bool found = false;
  const int wns[5] = {1, 2, 4, 8, 16};
  for (int wi = 0; wi < 5; ++wi) {
    const int wn = wns[wi], wk = 16 / wn;
    for (int ks = 1; ks <= std::min(ksteps, 64); ++ks) {
      int kpw = (ksteps + ks - 1) / ks;
      if (x_in_lds) {
        kpw = (kpw + 3) / 4 * 4;
        if (M * kpw * 32 * 2 > DEC_XS_BYTES) continue;
      }
      if ((int64_t)(ks - 1) * kpw >= ksteps) continue;
      const int kpw_wave = (kpw + wk - 1) / wk;
      for (int ntpw = 1; ntpw <= DEC_NT_MAX; ++ntpw) {
        const int ns = (ntiles + ntpw - 1) / ntpw;
        const int ntpw_real = (ntiles + ns - 1) / ns;
        const int per_wave_n = (ntpw_real + wn - 1) / wn;
        int nt_inst = 0;
        for (int i = 0; i < ninst; ++i)
          if (inst[i] >= per_wave_n) {
            nt_inst = inst[i];
            break;
          }
        if (nt_inst == 0) continue;
        const int64_t wgs = (int64_t)ks * ns;
        const int64_t rounds = (wgs + 255) / 256;
        // the CU's LDS gathers cover the workgroup's real tile-steps; the
        // padded per-wave share bounds the slowest wave
        const double decode =
            (double)rounds *
            (30.0 * passes * gfac * ((double)ntpw_real * kpw + 16.0 * kpw_wave * nt_inst) + 10000.0);
        const double partial = (double)ks * M * N * 8.0 / 2083.0;
        // every column slice reads all M rows of Xr over its k range again
        // (ns M K fp16 through the L2s, about 10 TB/s)
        const double xread = (double)ns * M * K * 2.2e-4;
        const double cost = decode + partial + xread;
        if (cost < best_cost - 1e-9) {
          best_cost = cost;
          best = DecodePlan{ks, ns, kpw, ntpw_real, wn, wk, nt_inst, x_in_lds ? 1 : 0, G};
          found = true;
        }
      }
    }
  }
  return found;
}

// The 4-bit kernel is compiled for more tile counts; the other widths share
// smaller instance sets. Both have 2 and 4 row groups per pass.
// For M <= 16 the rotation in the prologue saves a launch, but it bounds the
// workgroup's k range (the slice must fit DEC_XS_BYTES), which forces a
// k-split and its partial traffic on wide layers; the plan with a separate
// rotation pass competes with a penalty for that pass (a launch plus M x K
// fp16 read and written, in the model's units).
DecodePlan plan_decode(int32_t K, int32_t N, int64_t M, bool four_bits) {
  DecodePlan p{1, 1, K / 32, 1, 1, 16, four_bits ? 1 : 2, 0, 1};
  double cost = 1e300;
  if (M <= 16 && plan_decode_search(K, N, M, true, 1, four_bits, p, cost))
    cost -= 6000.0 + (double)M * K * 4.0 / 2083.0;
  else
    cost = 1e300;
  for (int G : {1, 2, 4})
    if (G == 1 || 16 * (G / 2) < M) plan_decode_search(K, N, M, false, G, four_bits, p, cost);
  return p;
}

struct PrefillLayout {
  size_t xr_off, w_off, part_off, total;
  int32_t chunk;
};
struct DecodeLayout {
  size_t xr_off, part_off, total;
  DecodePlan plan;
};

PrefillLayout prefill_layout(int32_t K, int32_t N, int64_t M) {
  PrefillLayout l;
  l.chunk = std::min<int32_t>(N, EXL3_MAX_CHUNK_COLS);
  l.xr_off = 0;
  // the rotated input in the GEMM's fragment order: rows padded to 32
  l.w_off = align256((size_t)((M + 31) / 32 * 32) * K * 2);
  l.part_off = l.w_off + align256((size_t)l.chunk * K * 2);
  // fp32 k-piece tiles of the GEMM's last round, for the widest slice and the
  // trailing one (the only two widths the slice loop uses)
  const int32_t last = N - (N - 1) / l.chunk * l.chunk;
  const size_t part = std::max(gemm_partial_bytes(l.chunk, (int32_t)M, K), gemm_partial_bytes(last, (int32_t)M, K));
  l.total = l.part_off + align256(part);
  return l;
}

// plan_decode is a pure function of (K, N, M, 4 bits or not); a small
// per-thread memo keeps its search off the per-call host path.
DecodePlan plan_decode_cached(int32_t K, int32_t N, int64_t M, bool four_bits) {
  struct Entry {
    int32_t K, N;
    int64_t M;
    bool four_bits;
    DecodePlan plan;
  };
  thread_local Entry memo[16];
  thread_local int used = 0, next = 0;
  for (int i = 0; i < used; ++i)
    if (memo[i].K == K && memo[i].N == N && memo[i].M == M && memo[i].four_bits == four_bits) return memo[i].plan;
  const DecodePlan p = plan_decode(K, N, M, four_bits);
  memo[next] = Entry{K, N, M, four_bits, p};
  next = (next + 1) % 16;
  if (used < 16) ++used;
  return p;
}

DecodeLayout decode_layout(int32_t K, int32_t N, int64_t M, int32_t bits) {
  DecodeLayout l;
  l.plan = plan_decode_cached(K, N, M, bits == 4);
  l.xr_off = 0;
  l.part_off = align256((size_t)M * K * 2);
  l.total = l.part_off + align256((size_t)l.plan.ks_count * M * N * 4);
  return l;
}

// Dequant-in-GEMM plan: row fragments per pass (1, 2, 4 or 8 fragments of
// 32 rows), 256-column units, and the split between whole units and K-split
// tail units, the combination that minimises the modelled time: rounds of
// 256 CUs, each as long as its workgroups' 16-k steps plus a fixed cost for
// the codebook load and the output stage, plus the tail's fp32 partials
// written and read back. The step costs (0.27, 0.32, 0.40 and 0.52 us for 1,
// 2, 4 and 8 fragments) are the slopes of whole-unit runs over K at the MLP
// geometries: the four waves' LDS gathers bound one fragment, the MFMAs and
// the shared operand loads the larger passes. The eight-wave kernel's step
// costs (0.28, 0.32 and 0.55 us for passes of 64, 128 and 256 rows): the
// 256-row slope of its whole-unit rounds at M = 2048, and the shorter passes
// scaled by their measured calls.
DqPlan plan_dq_rows(int32_t K, int32_t N, int64_t M, int nqb, bool whole, double& best, bool eight_waves = false) {
  static constexpr double kStepUs[9] = {0, 0.27, 0.32, 0, 0.40, 0, 0, 0, 0.52};
  static constexpr double kStepUs8[9] = {0, 0, 0.28, 0, 0.32, 0, 0, 0, 0.55};
  DqPlan p;
  p.nqb = nqb;
  const int R = 32 * nqb;
  p.passes = (int32_t)((M + R - 1) / R);
  p.pblocks = (N + 255) / 256;
  const int ksub = K / 16;
  const int64_t units = (int64_t)p.passes * p.pblocks;
  const double step_us = (eight_waves ? kStepUs8 : kStepUs)[nqb], wg_us = 3.0;
  auto rounds = [](int64_t wgs) { return (double)((wgs + 255) / 256); };
  best = 1e300;
  p.full = (int32_t)units;
  p.tail = 0;
  p.tail_ks = 1;
  p.ksub_per_piece = ksub;
  p.sk_steps = 0;
  p.sk_wgs = 0;
  const int64_t fr = units / 256;
  for (int64_t nf = std::max<int64_t>(0, fr - 1); nf <= fr; ++nf) {
    const int64_t full = nf * 256, tail = units - full;
    // k pieces are whole blocks of `align` 16-k steps: 4 (the kernels' loops
    // run 32-k steps in pairs), 8 for the eight-wave kernel's 64-row passes
    // (its x stages hold four 32-k steps); ksub is a multiple of 8
    const int align = eight_waves && nqb == 2 ? 8 : 4;
    for (int ks = 1; ks <= (whole ? 1 : std::min(ksub / align, 16)); ++ks) {
      if (tail == 0 && ks > 1) break;
      const int per = ((ksub + ks - 1) / ks + align - 1) / align * align;
      const int ks_eff = (ksub + per - 1) / per;
      double t = rounds(full) * (ksub * step_us + wg_us);
      if (ks_eff == 1) {
        t = rounds(full + tail) * (ksub * step_us + wg_us);
      } else {
        t += rounds(tail * ks_eff) * (per * step_us + wg_us) + (double)tail * ks_eff * R * 256 * 8.0 / 4e6;
      }
      if (t < best - 1e-9) {
        best = t;
        p.full = (int32_t)(ks_eff == 1 ? units : full);
        p.tail = (int32_t)(ks_eff == 1 ? 0 : tail);
        p.tail_ks = ks_eff;
        p.ksub_per_piece = ks_eff == 1 ? ksub : per;
        p.sk_steps = 0;
        p.sk_wgs = 0;
      }
    }
    // The eight-wave kernel's stream-K tail: the tail units' 32-k steps dealt
    // evenly to up to 256 workgroups (runs of whole blocks, at most one unit
    // long, so a run touches at most two units), one fp32 partial per unit
    // a run touches. Equal pieces per unit leave CUs idle when the tail units
    // times the pieces fall short of 256 (68 units x 3 pieces = 204).
    if (eight_waves && !whole && tail > 0 && tail <= 256) {
      const int ks32 = ksub / 2, al = align / 2;  // in 32-k steps
      const int64_t total = tail * ks32;
      const int per32 = (int)(((total + 255) / 256 + al - 1) / al * al);
      if (per32 <= ks32) {
        const int64_t wgs = (total + per32 - 1) / per32;
        // a run that crosses into a second unit refills its pipeline there:
        // one more fixed cost
        const double t = rounds(full) * (ksub * step_us + wg_us) + (2 * per32 * step_us + 2 * wg_us) +
                         (double)(wgs + tail) * R * 256 * 8.0 / 4e6;
        if (t < best - 1e-9) {
          best = t;
          p.full = (int32_t)full;
          p.tail = (int32_t)tail;
          p.tail_ks = 1;
          p.ksub_per_piece = 2 * per32;
          p.sk_steps = per32;
          p.sk_wgs = (int32_t)wgs;
        }
      }
    }
  }
  return p;
}

// The least modelled time over the row-fragment counts that leave no whole
// fragment of a pass empty (a pass of R rows serves M in ceil(M / R) passes).
// The eight-wave kernel takes the shortest pass of 64, 128 or 256 rows that
// covers M (256 above): its step is bound by the codebook gathers, which a
// second pass repeats, more than by the MFMAs and Xr reads a taller pass
// adds (K17408 x N5120, M = 256: one 256-row pass 74 us, two 128-row passes
// 83 us).
DqPlan plan_dq(int32_t K, int32_t N, int64_t M, bool whole = false, bool eight_waves = false) {
  DqPlan best_plan{};
  double best = 1e300;
  if (eight_waves) {
    const int nqb = M <= 64 ? 2 : M <= 128 ? 4 : 8;
    return plan_dq_rows(K, N, M, nqb, whole, best, true);
  }
  for (int nqb : {1, 2, 4, 8}) {
    if (nqb > 1 && 32 * (nqb / 2) >= M) break;
    double t;
    const DqPlan p = plan_dq_rows(K, N, M, nqb, whole, t, eight_waves);
    if (t < best - 1e-9) {
      best = t;
      best_plan = p;
    }
  }
  return best_plan;
}

struct DqLayout {
  size_t xf_off, part_off, total;
  DqPlan plan;
};

DqLayout dq_layout(int32_t K, int32_t N, int64_t M, bool whole = false, bool eight_waves = false) {
  DqLayout l;
  l.plan = plan_dq(K, N, M, whole, eight_waves);
  l.xf_off = 0;
  l.part_off = align256((size_t)((M + 31) / 32 * 32) * K * 2);
  l.total = l.part_off + align256(dq_partial_bytes(l.plan));
  return l;
}

}  // namespace

extern "C" {

const char* exl3_strerror(int status) {
  switch (status) {
    case EXL3_OK:
      return "ok";
    case EXL3_EINVAL:
    case EXL3_ESHAPE:
    case EXL3_ESCRATCH:
    case EXL3_EWIDTH:
    case EXL3_EHIP:
    case EXL3_EARCH:
      return g_msg[0] ? g_msg : "error";
    default:
      return "unknown status";
  }
}

}  // extern "C"

namespace {

// The kernel sequence of one call. At 4 bits the eight-wave dequant-GEMM
// takes the row counts where it measured fastest on both MLP geometries:
// from 33 rows on the fused side (the decode-GEMM below, whose cost steps up
// past 32 rows) and up to 1024 rows on the prefill side (reconstruct + GEMM
// above). The four-wave dequant-GEMM
// is slower at every row count measured and runs only when forced, as do the
// other sequences outside their ranges.
enum Route {
  kRouteDecode,
  kRouteReconstructGemm,
  kRouteDequantGemm,
  kRouteDequantGemmWhole,
  kRouteDequantGemm8,
  kRouteDequantGemm8Whole
};
constexpr int64_t kDqFusedMinRows = 33, kDqPrefillMaxRows = 1024;

Route route_of(int32_t bits, int64_t M, int32_t prefill_min_m, int variant) {
  switch (variant) {
    case kVariantFused:
      return kRouteDecode;
    case kVariantReconstructGemm:
      return kRouteReconstructGemm;
    case kVariantDequantGemm:
      return kRouteDequantGemm;
    case kVariantDequantGemmWhole:
      return kRouteDequantGemmWhole;
    case kVariantDequantGemm8:
      return kRouteDequantGemm8;
    case kVariantDequantGemm8Whole:
      return kRouteDequantGemm8Whole;
    default:
      break;
  }
  const bool dq_ok = bits == 4;
  const Route dq = kRouteDequantGemm8;
  if (use_prefill(M, prefill_min_m)) return dq_ok && M <= kDqPrefillMaxRows ? dq : kRouteReconstructGemm;
  return dq_ok && M >= kDqFusedMinRows ? dq : kRouteDecode;
}

size_t route_scratch_bytes(Route r, int32_t K, int32_t ncols, int64_t M, int32_t bits) {
  switch (r) {
    case kRouteReconstructGemm:
      return prefill_layout(K, ncols, M).total;
    case kRouteDequantGemm:
    case kRouteDequantGemmWhole:
    case kRouteDequantGemm8:
    case kRouteDequantGemm8Whole:
      return dq_layout(K, ncols, M, r == kRouteDequantGemmWhole || r == kRouteDequantGemm8Whole,
                       r == kRouteDequantGemm8 || r == kRouteDequantGemm8Whole)
          .total;
    default:
      return decode_layout(K, ncols, M, bits).total;
  }
}

// The layer over its leading ncols columns (ncols a multiple of 128, at most
// N), written to y with leading dimension ldy. Arguments are validated by the
// callers; scratch holds linear_cols_scratch_bytes(K, ncols, M, pm). The
// size does not depend on the width, so it covers the route taken at 4 bits
// and the one taken at the other widths (whose decode plans also differ).
size_t linear_cols_scratch_bytes(int32_t K, int32_t ncols, int64_t M, int32_t prefill_min_m,
                                 int variant = kVariantAuto) {
  return std::max(route_scratch_bytes(route_of(4, M, prefill_min_m, variant), K, ncols, M, 4),
                  route_scratch_bytes(route_of(3, M, prefill_min_m, variant), K, ncols, M, 3));
}

int linear_cols(const exl3_layer* L, const uint16_t* x, int64_t M, uint16_t* y, int64_t ldy, int32_t ncols,
                char* sb, int32_t prefill_min_m, hipStream_t stream, Marks* marks) {
  const int32_t K = L->K, N = L->N;
  const Route route = route_of(L->bits, M, prefill_min_m, marks ? marks->variant : kVariantAuto);
  if (route == kRouteDequantGemm || route == kRouteDequantGemmWhole || route == kRouteDequantGemm8 ||
      route == kRouteDequantGemm8Whole) {
    if (L->bits != 4) return fail(EXL3_ESHAPE, "the dequant-GEMM takes 4-bit codes only");
    const bool eight = route == kRouteDequantGemm8 || route == kRouteDequantGemm8Whole;
    const DqLayout l =
        dq_layout(K, ncols, M, route == kRouteDequantGemmWhole || route == kRouteDequantGemm8Whole, eight);
    uint16_t* xf = (uint16_t*)(sb + l.xf_off);
    float* part = (float*)(sb + l.part_off);
    EXL3_TRY(launch_had128_frag(x, xf, M, K, L->sign_k, eight, stream), "input rotation");
    EXL3_TRY(mark_begin(marks, kMarkDecode, stream), "event record");
    if (eight)
      EXL3_TRY(launch_dqgemm2(xf, L->codes, L->codebook, L->scale, L->sign_n, y, ldy, part, K, ncols, N / 16,
                              (int32_t)M, l.plan, stream),
               "dequant gemm");
    else
      EXL3_TRY(launch_dqgemm(xf, L->codes, L->codebook, L->scale, L->sign_n, y, ldy, part, K, ncols, N / 16,
                             (int32_t)M, l.plan, stream),
               "dequant gemm");
    EXL3_TRY(mark_end(marks, kMarkDecode, stream), "event record");
  } else if (route == kRouteReconstructGemm) {
    const PrefillLayout l = prefill_layout(K, ncols, M);
    uint16_t* xr = (uint16_t*)(sb + l.xr_off);
    uint16_t* wt = (uint16_t*)(sb + l.w_off);
    EXL3_TRY(launch_had128_frag(x, xr, M, K, L->sign_k, true, stream), "input rotation");
    for (int32_t n0 = 0; n0 < ncols; n0 += l.chunk) {
      const int32_t nc = std::min(l.chunk, ncols - n0);
      EXL3_TRY(mark_begin(marks, kMarkReconstruct, stream), "event record");
      EXL3_TRY(launch_reconstruct_nk(L->codes, L->codebook, L->scale, K, N, L->bits, n0, nc, wt, K, stream),
               "reconstruct");
      EXL3_TRY(mark_end(marks, kMarkReconstruct, stream), "event record");
      EXL3_TRY(launch_gemm_had(wt, xr, y, nc, (int32_t)M, K, ldy, n0, L->sign_n, (float*)(sb + l.part_off), stream,
                               marks),
               "gemm");
    }
  } else {
    const DecodeLayout l = decode_layout(K, ncols, M, L->bits);
    uint16_t* xr = (uint16_t*)(sb + l.xr_off);
    float* part = (float*)(sb + l.part_off);
    if (!l.plan.x_in_lds) EXL3_TRY(launch_had128(x, xr, M, K, L->sign_k, nullptr, stream), "input rotation");
    EXL3_TRY(mark_begin(marks, kMarkDecode, stream), "event record");
    EXL3_TRY(launch_decode_gemm(l.plan.x_in_lds ? x : xr, l.plan.x_in_lds ? L->sign_k : nullptr, L->codes,
                                L->codebook, part, K, ncols, N / 16, (int32_t)M, L->bits, l.plan, stream),
             "decode gemm");
    EXL3_TRY(mark_end(marks, kMarkDecode, stream), "event record");
    EXL3_TRY(launch_decode_finalize(part, l.plan.ks_count, L->scale, L->sign_n, y, ldy, (int32_t)M, ncols, stream),
             "decode finalize");
  }
  return EXL3_OK;
}

// Common call checks of exl3_linear and exl3_head_logits_argmax.
// own_scratch: the library supplies the scratch (the allocation-free entry
// point), so the caller's scratch argument is not checked.
int validate_call(const exl3_layer* L, const uint16_t* x, int64_t M, const void* y, const void* scratch,
                  int32_t prefill_min_m, bool own_scratch = false, int variant = kVariantAuto) {
  int st = validate_layer(L);
  if (st) return st;
  if (M < 0) return fail(EXL3_EINVAL, "M = %lld is negative", (long long)M);
  if (prefill_min_m < 0) return fail(EXL3_EINVAL, "prefill_min_m = %d is negative", prefill_min_m);
  // rows are padded to multiples of 32 in int32
  if (M > 0x7FFFFFE0) return fail(EXL3_EINVAL, "M = %lld is too large", (long long)M);
  if (M == 0) return EXL3_OK;
  if (!x || !y) return fail(EXL3_EINVAL, "x or the output is NULL");
  if (!own_scratch && !scratch) return fail(EXL3_EINVAL, "scratch is NULL");
  if (!aligned16(x) || !aligned16(y) || (!own_scratch && ((uintptr_t)scratch & 255u)))
    return fail(EXL3_EINVAL, "x and the output must be 16-byte aligned and scratch 256-byte aligned");
  // the prefill GEMM addresses the rotated input (M x K fp16) with 32-bit
  // byte offsets
  if (route_of(L->bits, M, prefill_min_m, variant) == kRouteReconstructGemm && M * L->K * 2 > (int64_t)UINT32_MAX)
    return fail(EXL3_ESHAPE, "M = %lld, K = %d: the prefill path needs M * K * 2 below 4 GiB", (long long)M, L->K);
  return EXL3_OK;
}

int64_t head_padded_width(int64_t n_valid, int64_t n) {
  const int64_t aligned = (n_valid + 127) / 128 * 128;
  return aligned < n ? aligned : n;
}

// The linear's scratch over the first n_pad columns, then the per-piece
// (order key, index) pairs of the argmax: two int32 arrays.
struct HeadLayout {
  size_t pk_off, pi_off, total;
};

HeadLayout head_layout(int32_t K, int32_t N, int64_t M, int64_t n_valid, int32_t prefill_min_m) {
  const int64_t n_pad = head_padded_width(n_valid, N);
  const size_t pairs = (size_t)M * head_argmax_items(n_pad);
  HeadLayout h;
  h.pk_off = align256(linear_cols_scratch_bytes(K, (int32_t)n_pad, M, prefill_min_m));
  h.pi_off = h.pk_off + align256(pairs * sizeof(int32_t));
  h.total = h.pi_off + align256(pairs * sizeof(int32_t));
  return h;
}

// Scratch of exl3_linear_noalloc: a file-scope device array, one copy on each
// GPU the library runs on, held until the process ends. Host code never
// passes the array's name to a kernel (on the host it is only a stand-in for
// the symbol): the device address comes from hipGetSymbolAddress, once per
// device with that device current, and is kept per device.
__device__ __align__(256) unsigned char scratch[EXL3_NOALLOC_SCRATCH_BYTES];

std::mutex g_noalloc_mu;
void* g_noalloc_ptr[64];  // device address of `scratch` per device index, once resolved

int noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(EXL3_EARCH, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_noalloc_mu);
  if (!g_noalloc_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p || ((uintptr_t)p & 255u)) return fail(EXL3_EHIP, "scratch symbol address %p is not 256-byte aligned", p);
    g_noalloc_ptr[dev] = p;
  }
  *out = g_noalloc_ptr[dev];
  return EXL3_OK;
}

}  // namespace

namespace exl3 {

int linear_entry(const exl3_layer* L, const uint16_t* x, int64_t M, uint16_t* y, void* scratch, size_t scratch_bytes,
                 int32_t prefill_min_m, hipStream_t stream, Marks* marks) {
  g_msg[0] = 0;
  const int variant = marks ? marks->variant : (int)kVariantAuto;
  int st = validate_call(L, x, M, y, scratch, prefill_min_m, false, variant);
  if (st || M == 0) return st;
  const size_t need = linear_cols_scratch_bytes(L->K, L->N, M, prefill_min_m, variant);
  if (scratch_bytes < need)
    return fail(EXL3_ESCRATCH, "scratch has %zu bytes; this call needs %zu", scratch_bytes, need);
  st = check_device();
  if (st) return st;
  return linear_cols(L, x, M, y, L->N, L->N, (char*)scratch, prefill_min_m, stream, marks);
}

size_t linear_variant_scratch_bytes(int32_t K, int32_t N, int64_t M, int32_t prefill_min_m, int variant) {
  if (K <= 0 || N <= 0 || K % 128 || N % 128 || M <= 0) return 0;
  return linear_cols_scratch_bytes(K, N, M, prefill_min_m, variant);
}

int logits_entry(const uint16_t* x, int64_t M, int32_t K, const uint16_t* w, int64_t w_rows, int64_t n_valid,
                 uint16_t* logits, int64_t ld_logits, int64_t* argmax, void* scratch, size_t scratch_bytes,
                 hipStream_t stream, Marks* marks) {
  g_msg[0] = 0;
  if (M < 0 || w_rows < 0) return fail(EXL3_EINVAL, "M = %lld, w_rows = %lld", (long long)M, (long long)w_rows);
  if (M > 0x7FFFFFFF || w_rows > 0x7FFFFFFF) return fail(EXL3_EINVAL, "M or w_rows too large");
  if (K <= 0 || K % 128 || K > (1 << 23))
    return fail(EXL3_ESHAPE, "K = %d must be a positive multiple of 128, at most 8388608", K);
  const int64_t n_pad = logits_padded_width(n_valid, w_rows);
  if (n_pad < 0)
    return fail(EXL3_EWIDTH, "n_valid = %lld must be in [1, w_rows = %lld]", (long long)n_valid, (long long)w_rows);
  if (ld_logits < n_pad)
    return fail(EXL3_EWIDTH, "ld_logits = %lld is below the padded width %lld", (long long)ld_logits,
                (long long)n_pad);
  if (M == 0) return EXL3_OK;
  if (!x || !w || !logits || !argmax || !scratch) return fail(EXL3_EINVAL, "a required pointer is NULL");
  if (!aligned16(x) || !aligned16(w) || ((uintptr_t)logits & 1) || ((uintptr_t)argmax & 7) ||
      ((uintptr_t)scratch & 255u))
    return fail(EXL3_EINVAL, "misaligned pointer");
  const size_t need = logits_scratch_bytes(M, K, n_valid, w_rows);
  if (scratch_bytes < need)
    return fail(EXL3_ESCRATCH, "scratch has %zu bytes; this call needs %zu", scratch_bytes, need);
  int st = check_device();
  if (st) return st;
  const int64_t items = logits_items(n_pad);
  int32_t* pk = (int32_t*)scratch;
  int32_t* pi = (int32_t*)((char*)scratch + align256((size_t)items * M * 4));
  uint16_t* xp = (uint16_t*)((char*)scratch + align256((size_t)items * M * 4) * 2);
  EXL3_TRY(launch_logits(x, (int32_t)M, K, w, n_valid, n_pad, logits, ld_logits, argmax, pk, pi, xp, stream, marks),
           "logits");
  return EXL3_OK;
}

int head_entry(const exl3_layer* L, const uint16_t* x, int64_t M, int64_t n_valid, uint16_t* logits,
               int64_t ld_logits, int64_t* argmax, void* scratch, size_t scratch_bytes, int32_t prefill_min_m,
               hipStream_t stream, Marks* marks) {
  g_msg[0] = 0;
  int st = validate_call(L, x, M, logits, scratch, prefill_min_m);
  if (st) return st;
  if (n_valid < 1 || n_valid > L->N)
    return fail(EXL3_EWIDTH, "n_valid = %lld must be in [1, N = %d]", (long long)n_valid, L->N);
  const int64_t n_pad = head_padded_width(n_valid, L->N);
  if (ld_logits < n_pad || ld_logits % 8)
    return fail(EXL3_EWIDTH, "ld_logits = %lld must be >= the padded width %lld and a multiple of 8",
                (long long)ld_logits, (long long)n_pad);
  if (M == 0) return EXL3_OK;
  if (!argmax || ((uintptr_t)argmax & 7u)) return fail(EXL3_EINVAL, "argmax is NULL or misaligned");
  const size_t need = exl3_head_scratch_bytes(L->K, L->N, M, n_valid, prefill_min_m);
  if (scratch_bytes < need)
    return fail(EXL3_ESCRATCH, "scratch has %zu bytes; this call needs %zu", scratch_bytes, need);
  st = check_device();
  if (st) return st;
  char* sb = (char*)scratch;
  const HeadLayout h = head_layout(L->K, L->N, M, n_valid, prefill_min_m);
  st = linear_cols(L, x, M, logits, ld_logits, (int32_t)n_pad, sb, prefill_min_m, stream, marks);
  if (st) return st;
  EXL3_TRY(launch_head_mask_argmax(logits, ld_logits, M, n_valid, n_pad, argmax, (int32_t*)(sb + h.pk_off),
                                   (int32_t*)(sb + h.pi_off), stream),
           "mask and argmax");
  return EXL3_OK;
}

}  // namespace exl3

extern "C" {

size_t exl3_linear_scratch_bytes(int32_t K, int32_t N, int64_t M, int32_t prefill_min_m) {
  if (K <= 0 || N <= 0 || K % 128 || N % 128 || M < 0) return 0;
  if (M == 0) return 0;
  return linear_cols_scratch_bytes(K, N, M, prefill_min_m);
}

int exl3_linear(const exl3_layer* L, const uint16_t* x, int64_t M, uint16_t* y, void* scratch, size_t scratch_bytes,
                int32_t prefill_min_m, void* stream_) {
  return exl3::linear_entry(L, x, M, y, scratch, scratch_bytes, prefill_min_m, (hipStream_t)stream_, nullptr);
}

int exl3_linear_noalloc(const exl3_layer* L, const uint16_t* x, int64_t M, uint16_t* y, int32_t prefill_min_m,
                        void* stream_) {
  g_msg[0] = 0;
  int st = validate_call(L, x, M, y, nullptr, prefill_min_m, true);
  if (st || M == 0) return st;
  const size_t need = exl3_linear_scratch_bytes(L->K, L->N, M, prefill_min_m);
  if (need > (size_t)EXL3_NOALLOC_SCRATCH_BYTES)
    return fail(EXL3_ESCRATCH, "this call needs %zu bytes of scratch; exl3_linear_noalloc holds %d (use exl3_linear "
                "with a caller-owned buffer)", need, EXL3_NOALLOC_SCRATCH_BYTES);
  st = check_device();
  if (st) return st;
  void* sb = nullptr;
  st = noalloc_scratch(&sb);
  if (st) return st;
  return linear_cols(L, x, M, y, L->N, L->N, (char*)sb, prefill_min_m, (hipStream_t)stream_, nullptr);
}

size_t exl3_head_scratch_bytes(int32_t K, int32_t N, int64_t M, int64_t n_valid, int32_t prefill_min_m) {
  if (K <= 0 || N <= 0 || K % 128 || N % 128 || M <= 0 || n_valid < 1 || n_valid > N) return 0;
  return head_layout(K, N, M, n_valid, prefill_min_m).total;
}

int exl3_head_logits_argmax(const exl3_layer* L, const uint16_t* x, int64_t M, int64_t n_valid, uint16_t* logits,
                            int64_t ld_logits, int64_t* argmax, void* scratch, size_t scratch_bytes,
                            int32_t prefill_min_m, void* stream_) {
  return exl3::head_entry(L, x, M, n_valid, logits, ld_logits, argmax, scratch, scratch_bytes, prefill_min_m,
                          (hipStream_t)stream_, nullptr);
}

int exl3_reconstruct(const exl3_layer* L, int32_t n0, int32_t n_count, uint16_t* w, int64_t ldw, int32_t layout,
                     void* stream_) {
  g_msg[0] = 0;
  int st = validate_layer(L);
  if (st) return st;
  if (!w) return fail(EXL3_EINVAL, "w is NULL");
  if (n0 < 0 || n_count < 0 || n0 % 16 || n_count % 16 || (int64_t)n0 + n_count > L->N)
    return fail(EXL3_ESHAPE, "slice [%d, %d + %d) must be 16-aligned and inside N = %d", n0, n0, n_count, L->N);
  if (layout != EXL3_LAYOUT_KN && layout != EXL3_LAYOUT_NK) return fail(EXL3_EINVAL, "unknown layout %d", layout);
  const int64_t minld = layout == EXL3_LAYOUT_KN ? n_count : L->K;
  if (ldw < minld || ldw % 8) return fail(EXL3_ESHAPE, "ldw = %lld must be >= %lld and a multiple of 8",
                                          (long long)ldw, (long long)minld);
  if (!aligned16(w)) return fail(EXL3_EINVAL, "w must be 16-byte aligned");
  if (n_count == 0) return EXL3_OK;
  st = check_device();
  if (st) return st;
  hipStream_t stream = (hipStream_t)stream_;
  if (layout == EXL3_LAYOUT_NK)
    EXL3_TRY(launch_reconstruct_nk(L->codes, L->codebook, L->scale, L->K, L->N, L->bits, n0, n_count, w, ldw,
                                   stream),
             "reconstruct");
  else
    EXL3_TRY(launch_reconstruct_kn(L->codes, L->codebook, L->scale, L->K, L->N, L->bits, n0, n_count, w, ldw, false,
                                   stream),
             "reconstruct");
  return EXL3_OK;
}

int exl3_decode_states(const exl3_layer* L, uint16_t* states, void* stream_) {
  g_msg[0] = 0;
  if (!L || !L->codes) return fail(EXL3_EINVAL, "layer or codes is NULL");
  int st = validate_codes_shape(L);
  if (st) return st;
  if (!states || !aligned16(states) || !aligned16(L->codes)) return fail(EXL3_EINVAL, "states NULL or misaligned");
  st = check_device();
  if (st) return st;
  EXL3_TRY(launch_reconstruct_kn(L->codes, nullptr, nullptr, L->K, L->N, L->bits, 0, L->N, states, L->N, true,
                                 (hipStream_t)stream_),
           "decode states");
  return EXL3_OK;
}

int had_r_128(const uint16_t* in, uint16_t* out, int64_t rows, int64_t cols, const uint16_t* sign_pre,
              const uint16_t* sign_post, void* stream_) {
  g_msg[0] = 0;
  if (rows < 0 || cols < 0) return fail(EXL3_EINVAL, "rows = %lld, cols = %lld", (long long)rows, (long long)cols);
  if (cols % 128) return fail(EXL3_ESHAPE, "cols = %lld is not a multiple of 128", (long long)cols);
  if (rows == 0 || cols == 0) return EXL3_OK;
  if (!in || !out) return fail(EXL3_EINVAL, "in or out is NULL");
  if (!aligned16(in) || !aligned16(out) || !aligned16(sign_pre) || !aligned16(sign_post))
    return fail(EXL3_EINVAL, "tensors must be 16-byte aligned");
  int st = check_device();
  if (st) return st;
  EXL3_TRY(launch_had128(in, out, rows, cols, sign_pre, sign_post, (hipStream_t)stream_), "had_r_128");
  return EXL3_OK;
}

int64_t logits_padded_width(int64_t n_valid, int64_t w_rows) {
  if (n_valid < 1 || n_valid > w_rows) return -1;
  const int64_t aligned = (n_valid + 127) / 128 * 128;
  return std::min(aligned, w_rows);
}

size_t logits_scratch_bytes(int64_t M, int32_t K, int64_t n_valid, int64_t w_rows) {
  const int64_t n_pad = logits_padded_width(n_valid, w_rows);
  if (n_pad < 0 || M < 0 || K < 0) return 0;
  const int64_t items = logits_items(n_pad);
  return align256((size_t)items * M * 4) * 2 + align256(logits_xperm_bytes(M, K));
}

int logits_pad_mask_argmax(const uint16_t* x, int64_t M, int32_t K, const uint16_t* w, int64_t w_rows,
                           int64_t n_valid, uint16_t* logits, int64_t ld_logits, int64_t* argmax, void* scratch,
                           size_t scratch_bytes, void* stream_) {
  return exl3::logits_entry(x, M, K, w, w_rows, n_valid, logits, ld_logits, argmax, scratch, scratch_bytes,
                            (hipStream_t)stream_, nullptr);
}

}  // extern "C"
