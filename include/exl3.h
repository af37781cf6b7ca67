/*
 * exl3.h -- C ABI of libexl3.so: an EXL3-style trellis-quantized linear layer
 * with 128-point Hadamard rotations, and the padded-width logits projection,
 * as hand-written HIP kernels for AMD Instinct MI355X (gfx950).
 *
 * Sources of the operations (the pages these functions follow):
 *   [P316] vLLM PR #316, "[EXL3] dispatch prefill-shaped GEMMs to
 *          reconstruct+hgemm": sections "Kernel measurements" (the unfused
 *          had_r_128 -> reconstruct[_slice] -> hgemm -> had_r_128 sequence),
 *          "Change" (in-op row-count dispatch, threshold 128, 0 disables;
 *          one reused fp16 scratch per geometry, <= 32768-column slices,
 *          336 MB bound), follow-up item 4 (Hadamard + reconstruct cost).
 *   [P314] vLLM PR #314, "[EXL3] allow CUDA-graph decode for dense
 *          checkpoints by priming exl3_gemm autotune": section "Problem"
 *          (a lazily allocated buffer on first call breaks graph capture;
 *          fail closed and name the failing condition), "Verification" (the
 *          checkpoint's lm_head is itself a trellis-quantized matrix).
 *   [P1046] pegainfer PR #1046, "perf(qwen35): align the logits GEMM width":
 *          Summary (round the decodable width up to a multiple of 128, clamp
 *          by the weight rows), the review follow-ups (pad columns forced to
 *          -inf after every logits GEMM, with nothing to do at an aligned width;
 *          GEMM and mask owned by one call so the GEMM is unreachable without
 *          the mask), Testing (248077 -> 248192 inside 248320 rows).
 *
 * Conventions for every function:
 *   - fp16 tensors are passed as uint16_t bit patterns.
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library
 *     never allocates, frees, synchronises the host, reads the environment or
 *     tunes by timing inside a call, so every call can be captured in a HIP
 *     graph. `stream` is a hipStream_t (NULL = the default stream); all work
 *     is enqueued on it in order.
 *   - Every function returns EXL3_OK (0) or an EXL3_E* status. Arguments are
 *     validated on the host before anything is launched (fail closed);
 *     exl3_strerror() names the failing condition. No C++ exception crosses
 *     the ABI.
 *   - Results are bit-identical from run to run (no float atomics; every
 *     reduction has a fixed order).
 *   - Calls on the same stream are ordered; calls on different streams that
 *     share a scratch buffer race.
 *
 * Stand-in weight format. The pages name the EXL3 trellis ("4-bit-class
 * trellis format", codebook selectors; 4-bit MLP layers and a 6-bit lm_head,
 * [P316] "Problem") without defining it, so this library fixes its own
 * documented stand-in, with b = `bits` per weight, 1 <= b <= 8:
 *   - The layer maps X (M x K) to Y (M x N); the stored weight W is K x N.
 *   - W is cut into 16 x 16 tiles over (k, n). Tile (kt, nt) is 8 b uint32
 *     words (32 b bytes: 128 at 4 bits) starting at word
 *     (kt * (N / 16) + nt) * 8 b of `codes` (K N b / 32 words in all).
 *   - Bit p (0 <= p < 256 b) of a tile is bit (p % 32) of word (p / 32).
 *   - Trellis step i (0..255) of a tile is the weight at k = 16 kt + i % 16,
 *     n = 16 nt + i / 16 (k runs fastest).
 *   - state(i) = sum_{t<16} bit((b i + t) mod 256 b) << t: a 16-bit shift
 *     register that takes in b new bits per step; the windows that run past
 *     the tile's last bit wrap round to its start (tail-biting).
 *   - W[k][n] = fp16_rne(codebook[state] * scale[n]) (the product of two fp16
 *     values is exact in fp32, so this is a single rounding).
 *   - The layer computes, per 128-element block and with H the natural-order
 *     (Sylvester) Hadamard matrix scaled by 1/sqrt(128):
 *         Xr = had(X * sign_k),  Yr = Xr . W,  Y = had(Yr) * sign_n,
 *     i.e. the pages' y = had_r_128(W . had_r_128(x)) with their W equal to
 *     the transpose of this W, plus random +-1 signs on both rotations.
 *   - Every width 1..8 uses the same 65536-entry codebook. The fused path
 *     shares each decoded tile between 1, 2 or 4 groups of 16 rows per pass
 *     at every width; 4 bits is compiled for more tile counts per wave.
 */
#ifndef EXL3_H
#define EXL3_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  EXL3_OK = 0,
  EXL3_EINVAL = 1,   /* NULL pointer where one is required, negative size */
  EXL3_ESHAPE = 2,   /* K or N not a multiple of 128, bits outside 1..8, misaligned slice, size beyond a limit */
  EXL3_ESCRATCH = 3, /* scratch smaller than the matching *_scratch_bytes() */
  EXL3_EWIDTH = 4,   /* n_valid < 1, n_valid > w_rows, ld_logits < padded width */
  EXL3_EHIP = 5,     /* a HIP runtime call or kernel launch failed */
  EXL3_EARCH = 6     /* the current device is not gfx950 */
};

/* A quantized layer. All pointers are device pointers.
 *   codes    : K * N / 8 uint32 words, tiles laid out as described above.
 *   codebook : 65536 fp16 values indexed by the 16-bit trellis state.
 *   scale    : N fp16 per-column scales.
 *   sign_k   : K fp16 values, each exactly +1.0 or -1.0 (only the sign bit
 *              is used), applied before the input rotation; NULL = all +1.
 *   sign_n   : N fp16 values, +-1.0, applied after the output rotation;
 *              NULL = all +1.
 *   K, N     : multiples of 128; bits in 1..8; the codes take K N bits / 8
 *              bytes, at most 4 GiB; K below 65536. */
typedef struct exl3_layer {
  const uint32_t *codes;
  const uint16_t *codebook;
  const uint16_t *scale;
  const uint16_t *sign_k;
  const uint16_t *sign_n;
  int32_t K;
  int32_t N;
  int32_t bits;
} exl3_layer;

/* Largest column slice the prefill path reconstructs at once [P316 "Change"]. */
#define EXL3_MAX_CHUNK_COLS 32768
/* Default row threshold of the prefill path [P316 "Change"]. */
#define EXL3_DEFAULT_PREFILL_MIN_M 128

/* y = layer(x) for x (M x K, row-major fp16) into y (M x N, row-major fp16).
 * Dispatch happens here, on the host, at call time [P316 "Change": the branch
 * must sit inside the op]: if prefill_min_m > 0 and M >= prefill_min_m the
 * prefill side runs, otherwise the fused side (prefill_min_m = 0: the fused
 * side for every M). Each side picks its kernels by width and row count:
 *   - prefill, reconstruct + GEMM (every width; 4 bits above 1024 rows): input
 *     rotation into scratch; then, per slice of at most EXL3_MAX_CHUNK_COLS
 *     columns, reconstruct the slice to fp16 into scratch and run the MFMA
 *     GEMM whose epilogue applies the output rotation and sign_n;
 *   - fused, decode-GEMM (widths other than 4; 4 bits up to 32 rows): a
 *     kernel that decodes every trellis tile once per pass of up to 64 rows
 *     and multiplies it with those rows -- for M <= 16 it also applies the
 *     input rotation itself, otherwise a rotation pass writes it to scratch
 *     first -- then an output-stage kernel that sums the split-K partials in
 *     a fixed order and applies the output rotation and sign_n;
 *   - dequant-GEMM (4 bits: 33 rows and up on the fused side, up to 1024 rows
 *     on the prefill side) [P316 follow-up item 4: dequantisation fused into
 *     the GEMM]: input rotation into scratch, then an MFMA GEMM of eight waves
 *     that decodes each trellis tile into its operand registers once per pass
 *     of 64, 128 or 256 rows (the shortest that covers M) while the pass's
 *     rows of the rotated input are staged in LDS, and applies scales, output
 *     rotation and sign_n in its epilogue; a K-split remainder of the work
 *     leaves fp32 partials that a fixup kernel sums in a fixed order before
 *     the same epilogue.
 * All three give y within the fp16 rounding of the same sums, not
 * bit-identical to each other. M = 0 is a no-op returning EXL3_OK.
 * Limits (EXL3_ESHAPE otherwise): K, N positive multiples of 128, K < 65536,
 * K * N / 2 (the packed codes) below 4 GiB, and on the reconstruct + GEMM
 * route M * K * 2 below 4 GiB; M at most 2^31 - 32 (EXL3_EINVAL otherwise).
 * scratch: device memory of at least
 *   exl3_linear_scratch_bytes(K, N, M, prefill_min_m) bytes, owned by the
 * caller and reusable across layers of the same geometry; its contents are
 * overwritten. x and y must not overlap each other or the scratch. */
int exl3_linear(const exl3_layer *layer, const uint16_t *x, int64_t M, uint16_t *y, void *scratch,
                size_t scratch_bytes, int32_t prefill_min_m, void *stream);

/* exl3_linear for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same dispatch, kernels and results (bit-identical to exl3_linear), with the
 * scratch held by the library instead of passed in -- a device array of
 * EXL3_NOALLOC_SCRATCH_BYTES (48 MiB) per GPU, kept until the process ends.
 * It covers every fused-path call below the default threshold at the MLP and
 * wide geometries (K5120 x N17408, K17408 x N5120, K5120 x N32768: at most
 * 34.3 MiB at M = 127); a call whose exl3_linear_scratch_bytes exceeds it
 * returns EXL3_ESCRATCH before any launch. The first call on a device looks
 * up the array's device address (hipGetSymbolAddress); no call allocates or
 * frees memory. Every call on one GPU uses that GPU's one array, and the
 * array keeps what the last call left (no kernel reads scratch it did not
 * write in the same call): calls that overlap on one GPU -- on different
 * streams, or from several threads -- race and must be ordered by the
 * caller. Other arguments, limits and statuses as exl3_linear. */
#define EXL3_NOALLOC_SCRATCH_BYTES (48 * 1024 * 1024)
int exl3_linear_noalloc(const exl3_layer *layer, const uint16_t *x, int64_t M, uint16_t *y, int32_t prefill_min_m,
                        void *stream);

/* Scratch needed by exl3_linear for this geometry, row count and threshold
 * (the path is chosen the same way), enough for a layer of any width 1..8.
 * Pure host function. Returns 0 for invalid shapes. */
size_t exl3_linear_scratch_bytes(int32_t K, int32_t N, int64_t M, int32_t prefill_min_m);

/* Reconstruct columns [n0, n0 + n_count) of W to fp16 [P316 "Kernel
 * measurements": reconstruct / reconstruct_slice], bit-exact with the format
 * definition above.
 *   layout = EXL3_LAYOUT_KN: w[k * ldw + j] = W[k][n0 + j], ldw >= n_count;
 *   layout = EXL3_LAYOUT_NK: w[j * ldw + k] = W[k][n0 + j], ldw >= K
 *            (the layout the prefill GEMM consumes).
 * n0 and n_count must be multiples of 16 with n0 + n_count <= N. */
#define EXL3_LAYOUT_KN 0
#define EXL3_LAYOUT_NK 1
int exl3_reconstruct(const exl3_layer *layer, int32_t n0, int32_t n_count, uint16_t *w, int64_t ldw,
                     int32_t layout, void *stream);

/* 128-point Walsh-Hadamard rotation of every 128-element block of every row
 * [P316 "Kernel measurements": had_r_128]:
 *   out[r][128b + i] = sign_post[128b + i] * (1/sqrt(128)) *
 *                      sum_j H[i][j] * sign_pre[128b + j] * in[r][128b + j]
 * with H[i][j] = (-1)^popcount(i & j). in/out are rows x cols row-major fp16;
 * cols must be a multiple of 128; sign vectors have cols entries (+-1.0, only
 * the sign bit is used) or are NULL (= +1). in == out (in place) is allowed.
 * Butterflies run in fp32; the result is rounded once to fp16. */
int had_r_128(const uint16_t *in, uint16_t *out, int64_t rows, int64_t cols, const uint16_t *sign_pre,
              const uint16_t *sign_post, void *stream);

/* Padded-width logits projection with pad masking and greedy selection
 * [P1046 Summary and review follow-ups]:
 *   n_pad = logits_padded_width(n_valid, w_rows);
 *   logits[m * ld_logits + n] = fp16(sum_k x[m][k] * w[n][k])  for n < n_valid
 *   logits[m * ld_logits + n] = -inf (0xFC00)                  for n_valid <= n < n_pad
 *   argmax[m] = the smallest n whose fp16 logit equals the row maximum, with
 *               NumPy's and torch's NaN rule: a NaN ranks above every number,
 *               so the first NaN wins; -0 equals +0. The pad columns come
 *               after every decodable one, so argmax[m] < n_valid always.
 * x: M x K row-major fp16; w: w_rows x K row-major fp16 (only rows < n_pad are
 * read; the GEMM runs over whole 128-row tiles up to n_pad); fp32 accumulation.
 * The GEMM and the mask are one call: there is no way to obtain padded logits
 * without the mask. K must be a positive multiple of 128, at most 8388608
 * (else EXL3_ESHAPE). scratch: at least
 * logits_scratch_bytes(M, K, n_valid, w_rows) bytes. M = 0 is a no-op. */
int logits_pad_mask_argmax(const uint16_t *x, int64_t M, int32_t K, const uint16_t *w, int64_t w_rows,
                           int64_t n_valid, uint16_t *logits, int64_t ld_logits, int64_t *argmax,
                           void *scratch, size_t scratch_bytes, void *stream);

/* min(round_up(n_valid, 128), w_rows), or -1 if n_valid < 1 or n_valid > w_rows
 * [P1046 Summary]. Pure host function. */
int64_t logits_padded_width(int64_t n_valid, int64_t w_rows);

/* Scratch needed by logits_pad_mask_argmax: per-wave (key, index) pairs and a
 * copy of x in MFMA fragment order. 0 for invalid arguments. Pure host
 * function. */
size_t logits_scratch_bytes(int64_t M, int32_t K, int64_t n_valid, int64_t w_rows);

/* Quantized output head: the padded-width logits projection of
 * logits_pad_mask_argmax with the weight held as a trellis layer instead of
 * dense fp16 rows [P314 "Verification": the checkpoint's lm_head is a
 * trellis-quantized matrix; P1046 Summary and review follow-ups: padded
 * width, pad columns -inf before selection]. With
 *   n_pad = min(round_up(n_valid, 128), N)   (logits_padded_width(n_valid, N))
 *   logits[m * ld_logits + n] = exl3_linear(layer, x)[m][n]   for n < n_valid
 *   logits[m * ld_logits + n] = -inf (0xFC00)                 for n_valid <= n < n_pad
 *   argmax[m] = the smallest n whose fp16 logit equals the row maximum (the
 *               NaN rule of logits_pad_mask_argmax; argmax[m] < n_valid).
 * Only the layer's first n_pad columns are computed (the output rotation
 * mixes columns inside 128-column blocks only, so they equal the full layer's
 * first n_pad columns); columns n_pad .. ld_logits - 1 of logits are left
 * untouched and codes of columns past n_pad are never read by the decode
 * path. Dispatch between the fused and the prefill path is exl3_linear's.
 * x: M x K fp16; logits: M rows with leading dimension ld_logits (a multiple
 * of 8, >= n_pad), 16-byte aligned; argmax: M int64, 8-byte aligned. scratch:
 * at least exl3_head_scratch_bytes(K, N, M, n_valid, prefill_min_m) bytes.
 * EXL3_EWIDTH for n_valid outside [1, N] or a bad ld_logits; other limits and
 * statuses as exl3_linear. M = 0 is a no-op. */
int exl3_head_logits_argmax(const exl3_layer *layer, const uint16_t *x, int64_t M, int64_t n_valid,
                            uint16_t *logits, int64_t ld_logits, int64_t *argmax, void *scratch,
                            size_t scratch_bytes, int32_t prefill_min_m, void *stream);

/* Scratch needed by exl3_head_logits_argmax: exl3_linear's scratch for the
 * first n_pad columns (enough for a layer of any width 1..8), then one
 * (int32 order key, int32 index) pair per row and 4096-column piece of the
 * argmax. Pure host function; 0 for invalid arguments or M = 0. */
size_t exl3_head_scratch_bytes(int32_t K, int32_t N, int64_t M, int64_t n_valid, int32_t prefill_min_m);

/* Test hook: states[k * N + n] = the 16-bit trellis state behind W[k][n]. */
int exl3_decode_states(const exl3_layer *layer, uint16_t *states, void *stream);

/* Human-readable text for a status; for EXL3_EHIP and validation failures it
 * names the condition of the most recent failing call on this thread. */
const char *exl3_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* EXL3_H */
