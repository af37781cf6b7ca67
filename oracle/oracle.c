/*
 * Plain CPU oracle for the EXL3-style trellis-quantized linear layer and the
 * padded-width logits projection.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or call
 * this file: only the test suite, the package smoke check and the benchmark's
 * CPU-baseline leg use it. It shares no code, header, table or constant with
 * the HIP library.
 *
 * Everything is computed in IEEE double precision, with a single direct
 * rounding to fp16 (round-to-nearest-even, written out below) at each point
 * where the unfused sequence of vLLM PR #316 ("Kernel measurements": the
 * had_r_128 -> reconstruct -> hgemm -> had_r_128 chain) materialises an fp16
 * tensor: the rotated input, the reconstructed weight, the GEMM output and the
 * rotated output. Build with -ffp-contract=off.
 *
 * Row-vector convention: X is M x K, the stored weight W is K x N,
 *     Xr = fp16(had128(X . diag(sK)))            (input rotation)
 *     W  = fp16(cb[state(k, n)] * scale[n])      (reconstruct)
 *     Yr = fp16(Xr . W)                          (GEMM, fp64 sum, k ascending)
 *     Y  = fp16(had128(Yr) . diag(sN))           (output rotation)
 * which is the pages' y = had_r_128(W . had_r_128(x)) with their W equal to the
 * transpose of this one and random +-1 signs on both rotations.
 *
 * The pages name the trellis format without defining it (vLLM PR #316, summary
 * and "Problem"; vLLM PR #314, "Problem"), so this project fixes a stand-in,
 * with b = bits per weight (1..8; the pages' MLP layers use 4, their lm_head
 * 6: vLLM PR #316, "Problem" and follow-up item 3):
 *   - 16x16 tiles over (k, n); tile (kt, nt) is 8b little-endian uint32 words
 *     (256 b bits) starting at word (kt * N/16 + nt) * 8b;
 *   - bit p (0 <= p < 256 b) of a tile is bit (p mod 32) of word (p / 32);
 *   - trellis step i (0..255) of the tile is the weight at row k = 16kt + i%16,
 *     column n = 16nt + i/16 (k runs fastest);
 *   - state(i) is the 16-bit window that starts at bit b*i, least significant
 *     bit first, wrapping from the tile's last bit to bit 0 (tail-biting): a
 *     shift register that takes in b new bits per step;
 *   - the weight is the fp16 codebook entry cb[state] times the fp16 scale of
 *     its column, rounded once to fp16.
 *
 * Parity pins for every function here live in tests/test_oracle_*.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- fp16 ---- */

/* fp16 bit pattern -> double (exact: every fp16 value is a double). */
static double h2d(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 31;
  int f = h & 1023;
  double v;
  if (e == 31) {
    v = f ? NAN : INFINITY;
  } else if (e == 0) {
    v = ldexp((double)f, -24);             /* subnormal: f * 2^-24 */
  } else {
    v = ldexp((double)(1024 + f), e - 25); /* (1 + f/1024) * 2^(e-15) */
  }
  return sign ? -v : v;
}

/* double -> fp16 bit pattern, one rounding, to nearest with ties to even.
 * ldexp/frexp scale by powers of two exactly and rint() rounds to the nearest
 * integer with ties to even under the default rounding mode. */
static uint16_t d2h(double v) {
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  double a = fabs(v);
  if (isnan(v)) return 0x7E00;
  if (a >= 65520.0) return sign | 0x7C00; /* 65520 is the midpoint of 65504 and 2^16: ties go up */
  if (a < ldexp(1.0, -14)) {
    /* subnormal range: quantum 2^-24; a result of 1024 is the smallest normal */
    double q = rint(ldexp(a, 24));
    return sign | (uint16_t)q;
  }
  int E;
  frexp(a, &E);           /* a = f * 2^E with f in [0.5, 1) */
  int e = E - 1;          /* a in [2^e, 2^(e+1)) */
  double q = rint(ldexp(a, 10 - e)); /* significand in units of 2^(e-10): [1024, 2048] */
  if (q == 2048.0) {
    q = 1024.0;
    e += 1;
  }
  return sign | (uint16_t)(((e + 15) << 10) | ((uint16_t)q - 1024));
}

static double *h2d_table(void) {
  double *t = (double *)malloc(65536 * sizeof(double));
  for (int i = 0; i < 65536; ++i) t[i] = h2d((uint16_t)i);
  return t;
}

void oracle_f16_to_f64(const uint16_t *in, double *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = h2d(in[i]);
}

void oracle_f64_to_f16(const double *in, uint16_t *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = d2h(in[i]);
}

/* ------------------------------------------------------------- trellis ---- */

/* Bit p of a tile (LSB-first words). */
static int tile_bit(const uint32_t *tile, int p) { return (tile[p >> 5] >> (p & 31)) & 1; }

/* state(i): the 16-bit window starting at bit bits*i, LSB first, wrapping at
 * the tile's 256*bits bits (tail-biting). */
static uint16_t tile_state(const uint32_t *tile, int bits, int i) {
  const int tile_len = 256 * bits;
  unsigned s = 0;
  for (int t = 0; t < 16; ++t) s |= (unsigned)tile_bit(tile, (bits * i + t) % tile_len) << t;
  return (uint16_t)s;
}

static uint16_t weight_state(const uint32_t *codes, int64_t N, int bits, int64_t k, int64_t n) {
  int64_t kt = k / 16, nt = n / 16;
  const uint32_t *tile = codes + (kt * (N / 16) + nt) * 8 * bits;
  int i = (int)((n % 16) * 16 + (k % 16));
  return tile_state(tile, bits, i);
}

/* states: K x N row-major, the trellis state behind every weight. */
void oracle_trellis_states(const uint32_t *codes, int64_t K, int64_t N, int64_t bits, uint16_t *states) {
#pragma omp parallel for schedule(static)
  for (int64_t k = 0; k < K; ++k)
    for (int64_t n = 0; n < N; ++n) states[k * N + n] = weight_state(codes, N, (int)bits, k, n);
}

/* W[k, n0 + j] for j < n_count, written K x n_count row-major. */
void oracle_reconstruct(const uint32_t *codes, const uint16_t *cb, const uint16_t *scale, int64_t K,
                        int64_t N, int64_t bits, int64_t n0, int64_t n_count, uint16_t *w) {
#pragma omp parallel for schedule(static)
  for (int64_t k = 0; k < K; ++k)
    for (int64_t j = 0; j < n_count; ++j) {
      int64_t n = n0 + j;
      double v = h2d(cb[weight_state(codes, N, (int)bits, k, n)]) * h2d(scale[n]); /* exact product */
      w[k * n_count + j] = d2h(v);
    }
}

/* ------------------------------------------------------------ hadamard ---- */

/* Entry (i, j) of the natural-order (Sylvester) Hadamard matrix of size 128. */
static int hadamard_sign(int i, int j) { return (__builtin_popcount((unsigned)(i & j)) & 1) ? -1 : 1; }

void oracle_hadamard_matrix(int8_t *h /* 128 x 128 */) {
  for (int i = 0; i < 128; ++i)
    for (int j = 0; j < 128; ++j) h[i * 128 + j] = (int8_t)hadamard_sign(i, j);
}

/* out = fp16(sign_post . (1/sqrt(128)) H (sign_pre . in)) per 128-element block
 * of each row, in double. A NULL sign vector means all +1. The matrix-vector
 * product is written out as the definition (128 terms per output). */
static void had_row(const double *in, const double *sign_pre, const double *sign_post, int64_t cols,
                    double *out) {
  const double norm = 1.0 / sqrt(128.0);
  for (int64_t b = 0; b < cols; b += 128) {
    for (int i = 0; i < 128; ++i) {
      double acc = 0.0;
      for (int j = 0; j < 128; ++j) {
        double v = in[b + j];
        if (sign_pre) v *= sign_pre[b + j];
        acc += hadamard_sign(i, j) * v;
      }
      acc *= norm;
      if (sign_post) acc *= sign_post[b + i];
      out[b + i] = acc;
    }
  }
}

void oracle_had128(const uint16_t *in, int64_t rows, int64_t cols, const uint16_t *sign_pre,
                   const uint16_t *sign_post, uint16_t *out) {
  double *sp = NULL, *sq = NULL;
  if (sign_pre) {
    sp = (double *)malloc(cols * sizeof(double));
    for (int64_t j = 0; j < cols; ++j) sp[j] = h2d(sign_pre[j]);
  }
  if (sign_post) {
    sq = (double *)malloc(cols * sizeof(double));
    for (int64_t j = 0; j < cols; ++j) sq[j] = h2d(sign_post[j]);
  }
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    double *a = (double *)malloc(cols * sizeof(double));
    double *b = (double *)malloc(cols * sizeof(double));
    for (int64_t j = 0; j < cols; ++j) a[j] = h2d(in[r * cols + j]);
    had_row(a, sp, sq, cols, b);
    for (int64_t j = 0; j < cols; ++j) out[r * cols + j] = d2h(b[j]);
    free(a);
    free(b);
  }
  free(sp);
  free(sq);
}

/* ---------------------------------------------------------- the layer ---- */

/* y[i, :] = layer(x[rows[i], :]) for the n_rows listed rows of x (M x K).
 * y is n_rows x N. Reconstructs the whole K x N weight once (fp16). */
void oracle_exl3_linear(const uint16_t *x, int64_t M, const int64_t *rows, int64_t n_rows,
                        const uint32_t *codes, const uint16_t *cb, const uint16_t *scale,
                        const uint16_t *sign_k, const uint16_t *sign_n, int64_t K, int64_t N,
                        int64_t bits, uint16_t *y) {
  (void)M;
  double *tab = h2d_table();
  uint16_t *w = (uint16_t *)malloc((size_t)K * N * sizeof(uint16_t));
  oracle_reconstruct(codes, cb, scale, K, N, bits, 0, N, w);
  double *sk = (double *)malloc(K * sizeof(double));
  double *sn = (double *)malloc(N * sizeof(double));
  for (int64_t k = 0; k < K; ++k) sk[k] = tab[sign_k[k]];
  for (int64_t n = 0; n < N; ++n) sn[n] = tab[sign_n[n]];

#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < n_rows; ++i) {
    const uint16_t *xr = x + rows[i] * K;
    double *xin = (double *)malloc(K * sizeof(double));
    double *xh = (double *)malloc(K * sizeof(double));
    double *acc = (double *)calloc(N, sizeof(double));
    double *yh = (double *)malloc(N * sizeof(double));
    double *yo = (double *)malloc(N * sizeof(double));
    /* input rotation, rounded to fp16 */
    for (int64_t k = 0; k < K; ++k) xin[k] = tab[xr[k]];
    had_row(xin, sk, NULL, K, xh);
    for (int64_t k = 0; k < K; ++k) xh[k] = tab[d2h(xh[k])];
    /* GEMM row: acc[n] = sum over k ascending of xh[k] * W[k, n] */
    for (int64_t k = 0; k < K; ++k) {
      const uint16_t *wk = w + k * N;
      double a = xh[k];
      for (int64_t n = 0; n < N; ++n) acc[n] += a * tab[wk[n]];
    }
    for (int64_t n = 0; n < N; ++n) yh[n] = tab[d2h(acc[n])];
    /* output rotation with the N-side signs, rounded to fp16 */
    had_row(yh, NULL, sn, N, yo);
    for (int64_t n = 0; n < N; ++n) y[i * N + n] = d2h(yo[n]);
    free(xin);
    free(xh);
    free(acc);
    free(yh);
    free(yo);
  }
  free(sk);
  free(sn);
  free(w);
  free(tab);
}

/* ------------------------------------------------------------- logits ---- */

/* Aligned width: the decodable width rounded up to a multiple of 128, clamped
 * by the number of weight rows (pegainfer PR #1046, Summary). */
int64_t oracle_padded_width(int64_t n_valid, int64_t w_rows) {
  int64_t aligned = (n_valid + 127) / 128 * 128;
  return aligned < w_rows ? aligned : w_rows;
}

/* Pad mask and greedy selection over one row of n_pad fp16 logits whose first
 * n_valid entries are set [P1046 review follow-ups: every pad column is -inf
 * before selection]: entries n_valid .. n_pad - 1 become -inf, and the result
 * is the smallest n whose value equals the row maximum (IEEE comparison, so
 * -0 equals +0). The pages do not say how a NaN logit is ranked; this follows
 * NumPy's and torch's argmax, where a NaN is the maximum and the first NaN
 * wins. */
static int64_t mask_and_select(uint16_t *row, int64_t n_valid, int64_t n_pad, const double *tab) {
  for (int64_t n = n_valid; n < n_pad; ++n) row[n] = 0xFC00; /* -inf */
  /* The first index of the largest value, where a NaN counts as larger than
   * every number (so the first NaN is selected): NumPy's and torch's argmax. */
  int64_t best = 0;
  double bv = tab[row[0]];
  for (int64_t n = 1; n < n_pad && !isnan(bv); ++n) {
    double v = tab[row[n]];
    if (isnan(v) || v > bv) {
      bv = v;
      best = n;
    }
  }
  return best;
}

/* For each listed row of x (M x K): logits over the padded width, then argmax.
 *   logits[i, n] = fp16(sum_k x[rows[i], k] * w[n, k])  for n < n_valid
 *   logits[i, n] = -inf                                 for n_valid <= n < n_pad
 * Rows of w at or beyond n_valid are never read: their values cannot reach the
 * result. argmax[i] is the smallest n whose fp16 logit equals the row maximum
 * (IEEE comparison; a NaN counts as the maximum, the first NaN wins). logits
 * is n_rows x n_pad. */
void oracle_logits(const uint16_t *x, int64_t M, const int64_t *rows, int64_t n_rows,
                   const uint16_t *w, int64_t w_rows, int64_t K, int64_t n_valid, uint16_t *logits,
                   int64_t *argmax) {
  (void)M;
  double *tab = h2d_table();
  int64_t n_pad = oracle_padded_width(n_valid, w_rows);
  for (int64_t i = 0; i < n_rows; ++i) {
    const uint16_t *xr = x + rows[i] * K;
    double *xd = (double *)malloc(K * sizeof(double));
    for (int64_t k = 0; k < K; ++k) xd[k] = tab[xr[k]];
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < n_valid; ++n) {
      const uint16_t *wn = w + n * K;
      double acc = 0.0;
      for (int64_t k = 0; k < K; ++k) acc += xd[k] * tab[wn[k]];
      logits[i * n_pad + n] = d2h(acc);
    }
    argmax[i] = mask_and_select(logits + i * n_pad, n_valid, n_pad, tab);
    free(xd);
  }
  free(tab);
}

/* ------------------------------------------------------ quantized head ---- */

/* The output head held as a trellis layer [P314 "Verification": the
 * checkpoint's lm_head is trellis-quantized; P1046 Summary and review
 * follow-ups]: for each listed row of x, the layer output (oracle_exl3_linear,
 * all N columns) is cut to its first n_pad = oracle_padded_width(n_valid, N)
 * columns, then pad-masked and selected as in oracle_logits. logits is
 * n_rows x n_pad; argmax has n_rows entries. */
void oracle_head_logits(const uint16_t *x, int64_t M, const int64_t *rows, int64_t n_rows,
                        const uint32_t *codes, const uint16_t *cb, const uint16_t *scale,
                        const uint16_t *sign_k, const uint16_t *sign_n, int64_t K, int64_t N,
                        int64_t bits, int64_t n_valid, uint16_t *logits, int64_t *argmax) {
  double *tab = h2d_table();
  int64_t n_pad = oracle_padded_width(n_valid, N);
  uint16_t *y = (uint16_t *)malloc((size_t)n_rows * N * sizeof(uint16_t));
  oracle_exl3_linear(x, M, rows, n_rows, codes, cb, scale, sign_k, sign_n, K, N, bits, y);
  for (int64_t i = 0; i < n_rows; ++i) {
    memcpy(logits + i * n_pad, y + i * N, (size_t)n_pad * sizeof(uint16_t));
    argmax[i] = mask_and_select(logits + i * n_pad, n_valid, n_pad, tab);
  }
  free(y);
  free(tab);
}
