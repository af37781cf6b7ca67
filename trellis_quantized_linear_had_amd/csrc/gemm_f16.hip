// Dense fp16 GEMM with fp32 accumulation on the MFMA units, with the output
// rotation fused into the epilogue (vLLM PR #316, "Kernel measurements": the
// hgemm between the two had_r_128 calls; follow-up item 2: hgemm against
// torch.mm at the MLP shapes).
//
//   D[p][q] = sum_k A[p][k] * B[q][k]     A = W^T slice (P x K), B = Xr (Q x K)
//   y[q][n0 + p] = fp16(sign_n[n0 + p] * (1/sqrt128) * sum_{p'} H[p][p'] D[p'][q])
//
// Computing the transpose (p = output column n, q = input row m) puts the
// 128-column rotation along the MFMA's row dimension, which a lane holds in
// registers: five of its seven butterfly stages run in registers and two
// cross lanes (16 and 32 apart).
//
// Tiling: 256 (p) x 256 (q) per workgroup, 64-wide k steps. 8 waves form
// 2 (p) x 4 (q); each owns 128 p-rows (one rotation block, 8
// v_mfma_f32_16x16x32_f16 row tiles) and 4 16-wide q tiles; two waves per
// SIMD. The 16x16x32 shape does the work of the 32x32x16 one with the same
// operand bytes per k, and under the chip's power limit it runs at a higher
// clock (measured: an MFMA loop on random data 1.86 vs 1.65 PFLOP/s). A k step
// is four half-steps h: k32 sub-step h / 2 on the p-tiles 4 (h % 2) .. + 3.
// A (W^T, shared by the 4 waves of a p half) goes from global memory straight
// into LDS (global_load_lds_dwordx4, no register staging), two stages, one
// barrier per k step. Inside a stage each 128-byte row is cut in 16-byte
// chunks XOR-swizzled by ((row >> 1) & 7): the LDS serves a 16-byte read 16
// lanes at a time over 64 banks, and the 16 lanes of a fragment read (16
// consecutive rows, one chunk) then hit 16 distinct bank groups. The swizzle
// is applied on the global side, because a direct-to-LDS load writes lane i's
// 16 bytes at base + 16 i. B (the rotated x, shared by only the 2 waves of a q
// quarter) does not pass through the LDS: the input rotation stores it in
// 16-row fragment order (had128_frag_kernel: 16 rows x 32 k per 1 KiB block,
// lane l holding row l % 16, k 8 (l / 16) .. + 8), so each wave loads its B
// fragments straight into registers, one contiguous 1 KiB per load
// instruction, one k step ahead.
//
// Tail balance: tiles are dealt to the 256 CUs in rounds. The largest
// multiple of 256 tiles runs whole; the k-steps of the remaining tiles are
// spread evenly over (up to) 256 workgroups, stream-K style, each writing an
// fp32 accumulator tile (in register order) per tile it touches, and a fixup
// kernel sums each tile's pieces in k order and runs the same rotation
// epilogue. Where those pieces would be short (at most an eighth of a tile's
// k-steps) the tail is dealt as 256 x 128 halves of its tiles (two 16-wide q
// tiles per wave): twice the k-steps per piece and half the partial bytes.
//
// Workgroup order is XCD-aware: workgroups are dispatched round-robin over
// the 8 XCDs, so workgroup w is given tile (w % 8) * ceil(T / 8) + w / 8. Each
// XCD then walks a contiguous run of tiles, q fastest: the 8 q-tiles that
// share one 256-row strip of W^T run together on one XCD and read it through
// that XCD's L2.
#include "common.h"
#include "epilogue.h"
#include "marks.h"

namespace exl3 {

#define G_BP 256
#define G_BQ 256
#define G_BK 64
#define G_PT 8   // 16-row p tiles per wave (128 rows)
#define G_QT 4   // 16-wide q tiles per wave (64 columns)
#define G_THREADS 512
#define G_STAGE (G_BP * G_BK)  // halves per stage (A only)
#define G_FRAG 512             // halves per 16 x 32 fragment block (1 KiB)
#define G_CUS 256

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ int swz_key(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int swz(int row, int chunk) { return row * G_BK + ((chunk ^ swz_key(row)) << 3); }

// Per-lane byte offsets of the 16-byte pieces one wave loads per k step from
// 32 consecutive rows of a row-major operand (8 rows, 1 KB per instruction):
// row wave_row0 + 8 i + lane / 8, source chunk (lane % 8) ^ key(row). Rows
// past the end re-read the last row (never stored).
__device__ __forceinline__ void lane_offsets(int64_t ld, int row_base, int rows_valid, int wave_row0, int lane,
                                             uint32_t (&off)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = wave_row0 + 8 * i + (lane >> 3);
    const int chunk = (lane & 7) ^ swz_key(r);
    const int gr = min(row_base + r, rows_valid - 1);
    off[i] = (uint32_t)(((int64_t)gr * ld + 8 * chunk) * 2);
  }
}

__device__ __forceinline__ void load_rows_lds(const uint16_t* __restrict__ g, int k0, const uint32_t (&off)[4],
                                              uint16_t* lds_stage, int wave_row0) {
  const char* base = reinterpret_cast<const char*>(g + k0);  // wave-uniform
#pragma unroll
  for (int i = 0; i < 4; ++i)
    __builtin_amdgcn_global_load_lds((const void*)(base + off[i]), (lds_void*)(lds_stage + (wave_row0 + 8 * i) * G_BK),
                                     16, 0, 0);
}

// One B fragment (16 bytes per lane) straight into registers. The load is
// issued through inline assembly so that the compiler does not track it: its
// waits cannot count register loads and the direct-to-LDS loads of A in one
// sequence and would fall back to waiting for all of them (vmcnt(0)) at the
// top of every k step. The kernel waits for these loads itself (wait_slot),
// with counts derived below from the loads each k step issues; the counts
// rely on vector memory loads returning in issue order, direct-to-LDS loads
// included.
__device__ __forceinline__ f16x8 load_frag(const uint16_t* p) {
  f16x8 v;
  asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(v) : "v"(p) : "memory");
  return v;
}

// Vector-memory loads one wave issues per k step, in issue order: B slot 0
// (the next k step's first k32 sub-step, QT fragments: QT 16-wide q tiles per
// wave), the 4 direct-to-LDS loads of the A stage after next (32 rows per
// wave, 8 rows per instruction), B slot 1 (its second k32 sub-step).
template <int QT>
struct GemmWaits {
  static constexpr int kBLoads = QT;
  static constexpr int kALoads = 4;
  static constexpr int kLoadsPerStep = 2 * kBLoads + kALoads;
  // Before half-step 0 slot 0 must have landed: issued after it, the A stage
  // and slot 1. Before half-step 2 slot 1 must have landed: issued after it,
  // this k step's refill of slot 0.
  static constexpr int kWaitSlot0 = kALoads + kBLoads;
  static constexpr int kWaitSlot1 = kBLoads;
  // Before the barrier the A stage (issued before slot 1's refill of the
  // previous k step) must have landed: issued after it, that refill and this
  // k step's refill of slot 0.
  static constexpr int kWaitStage = 2 * kBLoads;
  // Prologue, issued in steady-state order (A stage 0, slot 0, A stage 1,
  // slot 1): A stage 0 has landed once the loads after it are outstanding.
  static constexpr int kWaitPrologue = kBLoads + kALoads + kBLoads;
  static_assert(kWaitPrologue < 64 && kWaitSlot0 < kLoadsPerStep && kWaitSlot1 < kWaitSlot0 &&
                    kWaitStage < kLoadsPerStep,
                "vmcnt counts out of range (6 bits)");
  static_assert(kWaitPrologue == kLoadsPerStep, "the prologue issues one k step's loads after A stage 0");
};

// Waits until at most N vector-memory loads are outstanding. The slot's
// registers are named as read and written by the wait, so the compiler can
// neither move the MFMAs that read them above it nor reuse them while their
// load may still be in flight.
template <int N, int QT>
__device__ __forceinline__ void wait_slot(f16x8 (&slot)[QT]) {
  static_assert(QT == 4 || QT == 2, "one operand per fragment of the slot");
  if constexpr (QT == 4)
    asm volatile("s_waitcnt vmcnt(%4)" : "+v"(slot[0]), "+v"(slot[1]), "+v"(slot[2]), "+v"(slot[3]) : "n"(N)
                 : "memory");
  else
    asm volatile("s_waitcnt vmcnt(%2)" : "+v"(slot[0]), "+v"(slot[1]) : "n"(N) : "memory");
}

// Epilogue of one wave's 128 x 16 QT block: QT 16-wide q blocks.
template <int QT>
__device__ __forceinline__ void rotate_store(f32x4 (&acc)[G_PT][QT], int lane, int pw, int qw, int P, int Q,
                                             uint16_t* __restrict__ y, int64_t ldy, int32_t n0,
                                             const uint16_t* __restrict__ sign_n) {
#pragma unroll
  for (int j = 0; j < QT; ++j) {
    f32x4 blk[G_PT];
#pragma unroll
    for (int i = 0; i < G_PT; ++i) blk[i] = acc[i][j];
    rotate_store_block16(blk, lane, pw, qw + 16 * j, P, Q, y, ldy, n0, sign_n);
  }
}

// One accumulator tile in scratch: 512 threads x 32 QT floats, stored as
// 8 QT float4 columns of 512 (coalesced in both the writer and the fixup).
template <int QT>
__device__ __forceinline__ void store_partial(const f32x4 (&acc)[G_PT][QT], f32x4* __restrict__ dst) {
#pragma unroll
  for (int i = 0; i < G_PT; ++i)
#pragma unroll
    for (int j = 0; j < QT; ++j) dst[(i * QT + j) * G_THREADS + threadIdx.x] = acc[i][j];
}

// Slot of the partial of piece v for tail tile t: the (piece, tile) pairs in
// order. A tile boundary t nk inside a piece (not at its start) adds one pair,
// and the boundaries at piece starts are the t with units | t nk, i.e. the
// multiples of sdiv = units / gcd(nk, units): slot = v + t - t / sdiv.
__device__ __forceinline__ int partial_slot(int v, int t, int sdiv) { return v + t - t / sdiv; }

// Tail tile t -> tile index. Pieces v and v + nk / gcd(nk, units) sit at the
// same k offsets of tiles t and t + sdiv, so with grp = sdiv (the tail whole
// p-strips, a whole number of sdiv-strip groups) the order
// t = grp (sg tiles_q + q) + i  <->  (strip p0 + grp sg + i, column block q)
// gives the pieces in one phase tiles that share a W^T strip (same sg, i) or
// an x~ block (same q) at the same k step, read once through their XCD's L2.
// grp = 0: the tiles in plain order (with one column block they still share
// x~).
__device__ __forceinline__ int tail_tile(int t, int tile_base, int tiles_q, int grp) {
  if (grp == 0) return tile_base + t;
  const int i = t % grp, r = t / grp, q = r % tiles_q, sg = r / tiles_q;
  return (tile_base / tiles_q + grp * sg + i) * tiles_q + q;
}

// MODE 0: workgroup w computes tile tile_base + t (t in XCD order, t < count)
// over all of K and runs the rotation epilogue. MODE 1 (stream-K tail): the
// count items' k-steps, item-major, are dealt in runs of `units` to the
// workgroups (an item is a tail tile, or at QT = 2 one of its two 256 x 128
// halves: item t is half t % SPLIT of tail tile t / SPLIT); piece v covers
// [v units, (v + 1) units), at most two items (units <= K / G_BK), and writes
// one partial per item it touches (slot partial_slot(v, item)). Piece v is workgroup v: workgroups are dealt
// round-robin over the 8 XCDs, so pieces v and v + 8 j share an XCD, and
// with a phase period nk / gcd(nk, units) that is a multiple of 8 the pieces
// in one phase (the same k offsets at every step) all run on one XCD.
template <int MODE, int QT>
__device__ __forceinline__ void gemm_had_body(const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
                                              uint16_t* __restrict__ y, int32_t P, int32_t Q, int32_t K, int64_t ldy,
                                              int32_t n0, const uint16_t* __restrict__ sign_n, int32_t tile_base,
                                              int32_t count, int32_t units, int32_t sdiv, int32_t grp,
                                              f32x4* __restrict__ partial) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * G_STAGE];
  using W = GemmWaits<QT>;
  constexpr int BQ = 64 * QT;          // q extent of this launch's tiles
  constexpr int SPLIT = G_BQ / BQ;     // tail sub-tiles per whole tile (q halves at QT = 2)
  static_assert(MODE == 1 || QT == 4, "whole tiles are 256 x 256");

  const int tiles_q = (Q + G_BQ - 1) / G_BQ;
  const int nk_all = K / G_BK;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wp = wave & 1, wq = wave >> 1;
  const int lrow = lane & 15, lchunk = lane >> 4;

  f32x4 acc[G_PT][QT];
  // A fragments of one half-step (4 p tiles), two register sets; B fragments
  // of the two k32 sub-steps of one k step: slot t is refilled with the next
  // k step's sub-step t once this k step's last MFMAs reading it are issued
  f16x8 af[2][4], bq[2][QT];
  // A fragments of half-step h of stage `stage`: p tiles 4 (h % 2) .. + 3,
  // k32 sub-step h / 2 (chunks 4 (h / 2) .. + 3, one per 16-lane group)
  auto read_frags = [&](int stage, int h, int set) {
    const uint16_t* As = smem + stage * G_STAGE;
    const int ch = 4 * (h >> 1) + lchunk;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      af[set][i] = *reinterpret_cast<const f16x8*>(&As[swz(128 * wp + 16 * (4 * (h & 1) + i) + lrow, ch)]);
  };
  auto mfmas = [&](int set, int h) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < QT; ++j) {
        f32x4& d = acc[4 * (h & 1) + i][j];
        d = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[set][i], bq[h >> 1][j], d, 0, 0, 0);
      }
  };
  // Pins the order inside one half-step: the 4 A-fragment reads of the next
  // half-step go out between the first MFMAs, so they land under the rest.
  auto interleave = [&]() {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one DS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4 * QT - 4, 0);
  };
  // ... and with a slot refill in the half-step: its QT B loads go out
  // between the next MFMAs.
  auto interleave_loads = [&]() {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one DS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    }
#pragma unroll
    for (int k = 0; k < QT; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one VMEM read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4 * QT - 4 - QT, 0);
  };

  // acc = sum over k-steps [kb0, kb1) of one tile. Schedule per k step kb
  // (stage buffer b = (kb - kb0) & 1), half-steps h = 0..3:
  //   h = 0: wait for slot 0; read h = 1's A fragments; MFMAs;
  //   h = 1: read h = 2's A fragments; MFMAs; refill slot 0 (B(kb + 1, 0));
  //   h = 2: wait for slot 1; read h = 3's A fragments; MFMAs;
  //   h = 3: its A fragments are in registers; wait for this wave's A loads
  //   of stage kb+1, barrier (every wave is done reading buffer b and stage
  //   kb+1 has landed), issue the A loads of stage kb+2 into buffer b, read
  //   h = 0 of stage kb+1, then run h = 3's MFMAs, which cover the barrier and
  //   the fragment-read latency; refill slot 1 (B(kb + 1, 1)).
  // B loads past the range re-read the last k step (never used). Ends with a
  // barrier, so the stage buffers may be refilled at once.
  auto run_tile = [&](int p_base, int q_base, int kb0, int kb1) {
#pragma unroll
    for (int i = 0; i < G_PT; ++i)
#pragma unroll
      for (int j = 0; j < QT; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};
    uint32_t offa[4];
    lane_offsets(K, p_base, P, 32 * wave, lane, offa);
    // this wave's B blocks: q rows q_base + 64 wq + 16 j (clamped to the last
    // block; rows past Q are never stored)
    const int nqb = (Q + 15) / 16, kt32 = K / 32;
    const uint16_t* bsrc[QT];
#pragma unroll
    for (int j = 0; j < QT; ++j) {
      const int qb = min((q_base + 16 * QT * wq + 16 * j) / 16, nqb - 1);
      bsrc[j] = B + ((int64_t)qb * kt32 * 64 + lane) * 8;
    }
    auto load_b = [&](int kb, int t) {
#pragma unroll
      for (int j = 0; j < QT; ++j) bq[t][j] = load_frag(bsrc[j] + (int64_t)(2 * kb + t) * G_FRAG);
    };
    auto issue_loads = [&](int stage, int k0) { load_rows_lds(A, k0, offa, smem + stage * G_STAGE, 32 * wave); };
    const int nk = kb1 - kb0;
    if (nk <= 0) return;
    // Every k step issues the same loads in the same order, so the waits are
    // fixed counts: A loads of a stage past the range re-load the last k step
    // into a buffer no later k step reads. The prologue issues its loads in
    // the steady state's order: A stage 0, slot 0, A stage 1, slot 1.
    issue_loads(0, kb0 * G_BK);
    load_b(kb0, 0);
    issue_loads(1, (kb0 + min(1, nk - 1)) * G_BK);
    load_b(kb0, 1);
    // stage 0 landed (the loads after it may not have)
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(W::kWaitPrologue) : "memory");
    __syncthreads();
    read_frags(0, 0, 0);
    for (int kk = 0; kk < nk; ++kk) {
      const int b = kk & 1;
      const int kn = kb0 + min(kk + 1, nk - 1);  // the k step the B slots are refilled with
      wait_slot<W::kWaitSlot0>(bq[0]);
      read_frags(b, 1, 1);
      mfmas(0, 0);
      interleave();
      __builtin_amdgcn_sched_barrier(0);
      read_frags(b, 2, 0);
      mfmas(1, 1);
      load_b(kn, 0);
      interleave_loads();
      __builtin_amdgcn_sched_barrier(0);
      wait_slot<W::kWaitSlot1>(bq[1]);
      read_frags(b, 3, 1);
      mfmas(0, 2);
      interleave();
      __builtin_amdgcn_sched_barrier(0);
      // only slot 1's refill of the previous k step and slot 0's refill of
      // this one may be outstanding: this wave's A loads of stage kk+1 (issued
      // before them) have landed
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(W::kWaitStage) : "memory");
      __syncthreads();
      issue_loads(b, (kb0 + min(kk + 2, nk - 1)) * G_BK);
      if (kk + 1 < nk) read_frags(b ^ 1, 0, 0);
      mfmas(1, 3);
      load_b(kn, 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    // the last B loads (of the last k step again) must land before their
    // registers are reused: the compiler does not know they are in flight
    wait_slot<0>(bq[0]);
    wait_slot<0>(bq[1]);
  };

  if (MODE == 0) {
    const int per_xcd = (count + 7) / 8;
    const int t = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
    if (t >= count) return;  // whole workgroup (uniform)
    const int tile = tile_base + t;
    const int p_base = (tile / tiles_q) * G_BP, q_base = (tile % tiles_q) * G_BQ;
    run_tile(p_base, q_base, 0, nk_all);
    rotate_store(acc, lane, p_base + 128 * wp, q_base + 16 * QT * wq, P, Q, y, ldy, n0, sign_n);
  } else {
    const int total = count * nk_all;
    const int pieces = (total + units - 1) / units;
    const int v = (int)blockIdx.x;
    if (v >= pieces) return;  // whole workgroup (uniform)
    int unit = v * units;
    const int end = min(unit + units, total);
    for (int seg = 0; seg < 2 && unit < end; ++seg) {
      const int t = unit / nk_all, kb0 = unit - t * nk_all, kb1 = min(nk_all, kb0 + (end - unit));
      const int tile = tail_tile(t / SPLIT, tile_base, tiles_q, grp);
      run_tile((tile / tiles_q) * G_BP, (tile % tiles_q) * G_BQ + (t % SPLIT) * BQ, kb0, kb1);
      store_partial(acc, partial + (int64_t)partial_slot(v, t, sdiv) * (G_BP * BQ / 4));
      unit += kb1 - kb0;
    }
  }
}

// Whole 256 x 256 tiles (MODE 0) and the stream-K tail over whole tiles (MODE 1).
template <int MODE>
__global__ __launch_bounds__(G_THREADS) void gemm_had_kernel(const uint16_t* __restrict__ A,
                                                             const uint16_t* __restrict__ B,
                                                             uint16_t* __restrict__ y, int32_t P, int32_t Q,
                                                             int32_t K, int64_t ldy, int32_t n0,
                                                             const uint16_t* __restrict__ sign_n, int32_t tile_base,
                                                             int32_t count, int32_t units, int32_t sdiv,
                                                             int32_t grp, f32x4* __restrict__ partial) {
  gemm_had_body<MODE, 4>(A, B, y, P, Q, K, ldy, n0, sign_n, tile_base, count, units, sdiv, grp, partial);
}

// The stream-K tail over 256 x 128 halves of the tail tiles (count = 2 rem).
__global__ __launch_bounds__(G_THREADS) void gemm_had_tail_half_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, uint16_t* __restrict__ y, int32_t P, int32_t Q,
    int32_t K, int64_t ldy, int32_t n0, const uint16_t* __restrict__ sign_n, int32_t tile_base, int32_t count,
    int32_t units, int32_t sdiv, int32_t grp, f32x4* __restrict__ partial) {
  gemm_had_body<1, 2>(A, B, y, P, Q, K, ldy, n0, sign_n, tile_base, count, units, sdiv, grp, partial);
}

// Sums the k-pieces of one 128 (p) x 16 (q) block of a tail item (a tail
// tile, or at QT = 2 one of its 256 x 128 halves) in piece order and runs the
// rotation epilogue. One single-wave workgroup per (item, wave, 16-wide q
// block) spreads the partial reads over the CUs; the loads of two pieces are
// in flight together.
template <int QT>
__device__ __forceinline__ void gemm_fixup_body(const f32x4* __restrict__ partial, int32_t units, int32_t sdiv,
                                                int32_t grp, int32_t tile_base, int32_t P, int32_t Q, int32_t K,
                                                uint16_t* __restrict__ y, int64_t ldy, int32_t n0,
                                                const uint16_t* __restrict__ sign_n) {
  constexpr int BQ = 64 * QT, SPLIT = G_BQ / BQ;
  const int per_tile = (G_THREADS / 64) * QT;
  const int item = blockIdx.x / per_tile, wave = (blockIdx.x % per_tile) / QT, j = blockIdx.x % QT;
  const int tiles_q = (Q + G_BQ - 1) / G_BQ;
  const int tile = tail_tile(item / SPLIT, tile_base, tiles_q, grp);
  const int p_base = (tile / tiles_q) * G_BP, q_base = (tile % tiles_q) * G_BQ + (item % SPLIT) * BQ;
  const int lane = threadIdx.x;
  const int tid = 64 * wave + lane;  // the thread of the k-piece workgroup this lane stands for
  const int wp = wave & 1, wq = wave >> 1;
  // pieces of this tile: the ones whose unit runs overlap
  // [item nk, (item + 1) nk), in k order
  const int nk = K / G_BK;
  const int w_lo = item * nk / units, w_hi = ((item + 1) * nk - 1) / units;
  auto piece = [&](int w) { return partial + (int64_t)partial_slot(w, item, sdiv) * (G_BP * BQ / 4) + tid; };
  f32x4 a[G_PT];
  {
    const f32x4* src = piece(w_lo);
#pragma unroll
    for (int i = 0; i < G_PT; ++i) a[i] = src[(i * QT + j) * G_THREADS];
  }
  for (int w = w_lo + 1; w <= w_hi; w += 2) {
    const f32x4* s0 = piece(w);
    const f32x4* s1 = piece(min(w + 1, w_hi));
    f32x4 v0[G_PT], v1[G_PT];
#pragma unroll
    for (int i = 0; i < G_PT; ++i) {
      v0[i] = s0[(i * QT + j) * G_THREADS];
      v1[i] = s1[(i * QT + j) * G_THREADS];
    }
#pragma unroll
    for (int i = 0; i < G_PT; ++i) a[i] += v0[i];
    if (w + 1 <= w_hi) {
#pragma unroll
      for (int i = 0; i < G_PT; ++i) a[i] += v1[i];
    }
  }
  rotate_store_block16(a, lane, p_base + 128 * wp, q_base + 16 * QT * wq + 16 * j, P, Q, y, ldy, n0, sign_n);
}

__global__ __launch_bounds__(64) void gemm_fixup_kernel(const f32x4* __restrict__ partial, int32_t units,
                                                        int32_t sdiv, int32_t grp, int32_t tile_base, int32_t P,
                                                        int32_t Q, int32_t K, uint16_t* __restrict__ y, int64_t ldy,
                                                        int32_t n0, const uint16_t* __restrict__ sign_n) {
  gemm_fixup_body<4>(partial, units, sdiv, grp, tile_base, P, Q, K, y, ldy, n0, sign_n);
}

// The fixup of the half-tile tail: one item per 256 x 128 half.
__global__ __launch_bounds__(64) void gemm_fixup_half_kernel(const f32x4* __restrict__ partial, int32_t units,
                                                             int32_t sdiv, int32_t grp, int32_t tile_base, int32_t P,
                                                             int32_t Q, int32_t K, uint16_t* __restrict__ y,
                                                             int64_t ldy, int32_t n0,
                                                             const uint16_t* __restrict__ sign_n) {
  gemm_fixup_body<2>(partial, units, sdiv, grp, tile_base, P, Q, K, y, ldy, n0, sign_n);
}

// Round plan: `full` tiles (whole rounds of 256) run whole; the `rem` tiles
// after them are spread stream-K style, `units` k-steps per workgroup over
// `pieces` workgroups, when that beats one more whole round with idle CUs
// (rem <= 224); otherwise they also run whole. grp > 0 selects the grouped
// tail order (tail_tile). split = 2: when a piece would be at most an eighth
// of a whole tile's k-steps, the tail tiles are dealt as 256 x 128 halves
// instead (twice the k-steps per piece, half the partial bytes per piece):
// the partials' round trip is then what the tail costs beyond its MFMAs, and
// halving it outweighs the half tile's lower MFMA rate, which decides at
// longer pieces.
struct GemmPlan {
  int tiles, full, rem, split, units, pieces, sdiv, slots, grp;
};

static GemmPlan gemm_plan(int32_t P, int32_t Q, int32_t K) {
  GemmPlan g;
  g.tiles = ((P + G_BP - 1) / G_BP) * ((Q + G_BQ - 1) / G_BQ);
  g.full = g.tiles / G_CUS * G_CUS;
  g.rem = g.tiles - g.full;
  g.split = 1;
  g.units = 0;
  g.pieces = 0;
  g.sdiv = 1;
  g.slots = 0;
  g.grp = 0;
  const int nk = K / G_BK;
  if (g.rem > 0 && g.rem <= 224 && nk >= 2) {
    const int64_t units_whole = ((int64_t)g.rem * nk + G_CUS - 1) / G_CUS;
    if (2 * g.rem <= G_CUS && 8 * units_whole <= nk) g.split = 2;
    const int sub = g.rem * g.split;  // tail items (tiles or halves)
    const int64_t total = (int64_t)sub * nk;
    g.units = (int)((total + G_CUS - 1) / G_CUS);  // <= nk because sub <= G_CUS
    g.pieces = (int)((total + g.units - 1) / g.units);
    int a = nk, b = g.units;  // gcd
    while (b) {
      const int r = a % b;
      a = b;
      b = r;
    }
    g.sdiv = g.units / a;
    const int t_last = sub - 1;
    g.slots = g.pieces + t_last - t_last / g.sdiv;  // one past the last slot
    const int tiles_q = (Q + G_BQ - 1) / G_BQ;
    if (g.split == 1 && g.full % tiles_q == 0 && g.rem % (tiles_q * g.sdiv) == 0) g.grp = g.sdiv;
  } else {
    g.full = g.tiles;
    g.rem = 0;
  }
  return g;
}

size_t gemm_partial_bytes(int32_t P, int32_t Q, int32_t K) {
  const GemmPlan g = gemm_plan(P, Q, K);
  return (size_t)g.slots * G_BP * (G_BQ / g.split) * sizeof(float);
}

hipError_t launch_gemm_had(const uint16_t* A, const uint16_t* B, uint16_t* y, int32_t P, int32_t Q, int32_t K,
                           int64_t ldy, int32_t n0, const uint16_t* sign_n, float* partial, hipStream_t stream,
                           Marks* marks) {
  const GemmPlan g = gemm_plan(P, Q, K);
  f32x4* part = reinterpret_cast<f32x4*>(partial);
  if (g.full > 0) {
    hipError_t e = mark_begin(marks, kMarkGemm, stream);
    if (e != hipSuccess) return e;
    gemm_had_kernel<0><<<8 * ((g.full + 7) / 8), G_THREADS, 0, stream>>>(A, B, y, P, Q, K, ldy, n0, sign_n, 0, g.full,
                                                                         0, 1, 0, part);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = mark_end(marks, kMarkGemm, stream);
    if (e != hipSuccess) return e;
  }
  if (g.rem > 0) {
    const unsigned grid = 8 * ((g.pieces + 7) / 8);
    // fixup: one single-wave workgroup per (tail item, wave, 16-wide q block)
    const unsigned fix = (unsigned)(g.rem * g.split) * (G_THREADS / 64) * (G_QT / g.split);
    if (g.split == 1) {
      gemm_had_kernel<1><<<grid, G_THREADS, 0, stream>>>(A, B, y, P, Q, K, ldy, n0, sign_n, g.full, g.rem, g.units,
                                                         g.sdiv, g.grp, part);
      gemm_fixup_kernel<<<fix, 64, 0, stream>>>(part, g.units, g.sdiv, g.grp, g.full, P, Q, K, y, ldy, n0, sign_n);
    } else {
      gemm_had_tail_half_kernel<<<grid, G_THREADS, 0, stream>>>(A, B, y, P, Q, K, ldy, n0, sign_n, g.full,
                                                                2 * g.rem, g.units, g.sdiv, g.grp, part);
      gemm_fixup_half_kernel<<<fix, 64, 0, stream>>>(part, g.units, g.sdiv, g.grp, g.full, P, Q, K, y, ldy, n0,
                                                     sign_n);
    }
  }
  return hipGetLastError();
}

}  // namespace exl3
