/*
 * hbl_oracle.c -- plain CPU oracle for the H-BitLinear forward of BitNet v2.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously-correct
 * reference that the HIP path is checked against.  Only the test suite, the
 * smoke check and the CPU-baseline leg of the benchmark may load it.  It
 * shares no code, header, table or constant with the GPU library.
 *
 * Source of every formula: the architecture write-up of
 * "BitNet v2: Native 4-bit Activations with Hadamard Transformation for
 * 1-bit LLMs" (paper-graph-ui.vercel.app, §3.4 "Detailed, Sentence-Based
 * Technical Breakdown"), cited below as [BNv2 §3.4 <subsection>, Eq. n].
 *
 * Precision policy.
 *   - The Hadamard transform is evaluated in fp64 (radix-2 butterflies on
 *     exactly-widened inputs, one final 1/sqrt(n) scale) and rounded once to
 *     fp32: that fp32 vector is the tensor X_r the quantizer sees.
 *   - Sums of absolute values (beta, alpha) are accumulated in fp64.
 *   - The quantizer's decision arithmetic (the scale factor, the product
 *     x*f, round-half-even, clip) is evaluated in fp32, the precision the
 *     GPU kernels decide in, so that both sides round the same quantity.
 *   - The integer matmul is exact (int64 accumulation, checked to fit int32).
 *   - Compile with -ffp-contract=off: no fused multiply-adds anywhere.
 *
 * Readings of points the pages leave open (also listed in the design notes):
 *   eps = 1e-5f for weights and activations; "round" is round-half-to-even;
 *   the per-token scale factor f = Qmax/(stat + eps) is formed once per row;
 *   the dequantisation factor uses the statistic without eps (gamma/127,
 *   beta/sqrt(7)); H is in natural (Sylvester) order, applied per token row;
 *   alpha is one scalar per weight matrix; Y[M][N] = Xq[M][K] * Wq[N][K]^T.
 *
 * Packed layouts (defined here, bit-exactly; the GPU library must match):
 *   ternary weights: uint32 [N][K/16]; word w of row n holds k = 16w..16w+15;
 *       weight j = 4s + b (s,b in 0..3) sits at bits [8b+2s, 8b+2s+2) as the
 *       unsigned value c = q + 1 in {0,1,2} (3 never occurs).
 *   INT4 codes: uint32 [M][K/8]; word w of row m holds k = 8w..8w+7;
 *       code j = 4h + b (h in 0..1, b in 0..3) sits at bits [8b+4h, 8b+4h+4)
 *       as a two's-complement nibble.
 *   INT8 codes: int8 [M][K], natural order.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fopenmp -shared -fPIC
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define HBO_EPS 1e-5f /* the pages' epsilon has no printed value; reading */

/* dtype codes understood by this oracle */
#define HBO_F32 0
#define HBO_BF16 1

/* ------------------------------------------------------------------ */
/* scalar helpers                                                      */
/* ------------------------------------------------------------------ */

/* bf16 -> fp32 is exact: the bf16 bits are the top half of the fp32 bits. */
static float bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* fp32 -> bf16, round to nearest, ties to even (finite inputs). */
uint16_t hbo_f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7fffu + lsb;
  return (uint16_t)(u >> 16);
}

static float load_elem(const void *x, int dtype, int64_t i) {
  if (dtype == HBO_BF16) return bf16_to_f32(((const uint16_t *)x)[i]);
  return ((const float *)x)[i];
}

/* RoundClip(X, a, b) = min(max(round(X), a), b)  [BNv2 §3.4 "Weight
 * Quantization", Eq. 2]; round = nearest, ties to even (rintf in the default
 * rounding mode). */
static float round_clip(float v, float a, float b) {
  float r = rintf(v);
  if (r < a) r = a;
  if (r > b) r = b;
  return r;
}

static int is_pow2(int64_t n) { return n > 0 && (n & (n - 1)) == 0; }

/* ------------------------------------------------------------------ */
/* Hadamard transform  [BNv2 §3.4 "The Hadamard Transformation",       */
/* Eq. 3-6]                                                            */
/* ------------------------------------------------------------------ */

/* In-place unnormalised Walsh-Hadamard transform of v[0..n), natural
 * (Sylvester) order: applies H~_m where H~_0 = (1) and
 * H~_m = [[H~_{m-1}, H~_{m-1}], [H~_{m-1}, -H~_{m-1}]].  One radix-2 stage
 * per power of two h = 1, 2, 4, ..., n/2: the pair (v[j], v[j+h]) becomes
 * (v[j] + v[j+h], v[j] - v[j+h]).  Returns the number of additions and
 * subtractions performed (n * log2 n). */
int64_t hbo_fwht_f64(double *v, int64_t n) {
  int64_t ops = 0;
  for (int64_t h = 1; h < n; h *= 2) {
    for (int64_t i = 0; i < n; i += 2 * h) {
      for (int64_t j = i; j < i + h; j++) {
        double a = v[j];
        double b = v[j + h];
        v[j] = a + b;
        v[j + h] = a - b;
        ops += 2;
      }
    }
  }
  return ops;
}

/* Y = Hadamard(X) row by row, normalised: each row of length K = 2^m is
 * multiplied by H_m = 2^{-m/2} H~_m  (the 1/sqrt(2) of every recursion level
 * in Eq. 5 collected into one factor).  y is fp64 [M][K]. */
int hbo_hadamard(const void *x, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                 double *y) {
  if (!is_pow2(K) || ldx < K || M < 0) return 2;
  const double scale = 1.0 / sqrt((double)K);
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; m++) {
    double *row = y + m * K;
    for (int64_t k = 0; k < K; k++) row[k] = (double)load_elem(x, x_dtype, m * ldx + k);
    hbo_fwht_f64(row, K);
    for (int64_t k = 0; k < K; k++) row[k] = row[k] * scale;
  }
  return 0;
}

/* ------------------------------------------------------------------ */
/* Per-token activation quantizers  [BNv2 §3.4 "INT8 Quantization",     */
/* Eq. 7; "INT4 Quantization", Eq. 8]                                  */
/* ------------------------------------------------------------------ */

/* Quantises one fp32 row xr[0..K) (the tensor X_r of Eq. 9).
 *   INT8: gamma = max|x|; q = RoundClip(127/(gamma+eps) * x, -128, 127);
 *         dequantisation factor s = gamma/127.
 *   INT4: beta = mean|x|;  q = RoundClip(sqrt(7)/(beta+eps) * x, -8, 7);
 *         dequantisation factor s = beta/sqrt(7).
 * Writes q[0..K) as int8 and returns s; *rowsum = sum of the codes. */
static float quantize_row(const float *xr, int64_t K, int bits, int8_t *q,
                          int32_t *rowsum) {
  float f, s, lo, hi;
  if (bits == 8) {
    float gamma = 0.0f;
    for (int64_t k = 0; k < K; k++) {
      float a = fabsf(xr[k]);
      if (a > gamma) gamma = a;
    }
    f = 127.0f / (gamma + HBO_EPS);
    s = gamma / 127.0f;
    lo = -128.0f;
    hi = 127.0f;
  } else {
    double sum = 0.0;
    for (int64_t k = 0; k < K; k++) sum += fabs((double)xr[k]);
    float beta = (float)(sum / (double)K);
    const float sqrt7 = (float)sqrt(7.0);
    f = sqrt7 / (beta + HBO_EPS);
    s = beta / sqrt7;
    lo = -8.0f;
    hi = 7.0f;
  }
  int64_t total = 0;
  for (int64_t k = 0; k < K; k++) {
    float v = round_clip(xr[k] * f, lo, hi);
    q[k] = (int8_t)v;
    total += (int64_t)q[k];
  }
  *rowsum = (int32_t)total;
  return s;
}

/* INT4 packing: code j = 4h + b of each 8-code group at bits [8b+4h, +4). */
void hbo_pack_int4(const int8_t *q, int64_t M, int64_t K, uint32_t *packed) {
  for (int64_t m = 0; m < M; m++)
    for (int64_t w = 0; w < K / 8; w++) {
      uint32_t word = 0;
      for (int j = 0; j < 8; j++) {
        int h = j / 4, b = j % 4;
        uint32_t nib = (uint32_t)(q[m * K + 8 * w + j]) & 0xfu;
        word |= nib << (8 * b + 4 * h);
      }
      packed[m * (K / 8) + w] = word;
    }
}

void hbo_unpack_int4(const uint32_t *packed, int64_t M, int64_t K, int8_t *q) {
  for (int64_t m = 0; m < M; m++)
    for (int64_t w = 0; w < K / 8; w++) {
      uint32_t word = packed[m * (K / 8) + w];
      for (int j = 0; j < 8; j++) {
        int h = j / 4, b = j % 4;
        int nib = (int)((word >> (8 * b + 4 * h)) & 0xfu);
        q[m * K + 8 * w + j] = (int8_t)(nib >= 8 ? nib - 16 : nib);
      }
    }
}

/* ------------------------------------------------------------------ */
/* Normalisation layer of H-BitLinear  [BNv2 §3.4 "H-BitLinear: The    */
/* Composite Layer", Eq. 9: X_r = Hadamard(LN(X)), LN = RMSNorm]       */
/* ------------------------------------------------------------------ */

/* RMSNorm of one row, in fp64: t[k] = x[k] * r * g[k] with
 * r = 1 / sqrt(mean_j x[j]^2 + eps) and g the per-channel gain (NULL: a
 * gain of one).  The pages name RMSNorm without printing it; this is the
 * usual root-mean-square normalisation, with the library's eps. */
static void rmsnorm_row_f64(const void *x, int x_dtype, int64_t off, int64_t K,
                            const float *gain, double *t) {
  double ss = 0.0;
  for (int64_t k = 0; k < K; k++) {
    double v = (double)load_elem(x, x_dtype, off + k);
    t[k] = v;
    ss += v * v;
  }
  const double r = 1.0 / sqrt(ss / (double)K + (double)HBO_EPS);
  for (int64_t k = 0; k < K; k++) t[k] = t[k] * r * (gain ? (double)gain[k] : 1.0);
}

/* X -> (codes, scales, rowsum), optionally through the normalisation layer
 * (norm != 0, gain nullable) and the rotation (hadamard != 0):
 *   t   = norm ? RMSNorm(x) : x            (fp64, exact widening of x)
 *   X_r = hadamard ? H t : t, rounded once to fp32
 * then the quantiser of Eq. 7 or Eq. 8 on X_r.
 * codes: int8 [M][K] for bits = 8, uint32 [M][K/8] (INT4 layout) for bits = 4.
 * xr_out (nullable): the fp32 values that were quantised, [M][K].
 * Returns 0, or 2 for a bad shape / mode. */
static int quantize_rows(const void *x, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                         int norm, const float *gain, int hadamard, int bits, void *codes,
                         float *scales, int32_t *rowsum, float *xr_out) {
  if (M < 0 || K <= 0 || ldx < K || (bits != 8 && bits != 4)) return 2;
  if (hadamard && !is_pow2(K)) return 2;
  if (bits == 4 && K % 8 != 0) return 2;
  const double scale = 1.0 / sqrt((double)K);
#pragma omp parallel
  {
    double *t = (double *)malloc((size_t)K * sizeof(double));
    float *xr = (float *)malloc((size_t)K * sizeof(float));
    int8_t *q = (int8_t *)malloc((size_t)K);
#pragma omp for schedule(static)
    for (int64_t m = 0; m < M; m++) {
      if (norm) {
        rmsnorm_row_f64(x, x_dtype, m * ldx, K, gain, t);
      } else {
        for (int64_t k = 0; k < K; k++) t[k] = (double)load_elem(x, x_dtype, m * ldx + k);
      }
      if (hadamard) {
        hbo_fwht_f64(t, K);
        for (int64_t k = 0; k < K; k++) xr[k] = (float)(t[k] * scale);
      } else {
        for (int64_t k = 0; k < K; k++) xr[k] = (float)t[k];
      }
      if (xr_out) memcpy(xr_out + m * K, xr, (size_t)K * sizeof(float));
      int32_t rs;
      float s = quantize_row(xr, K, bits, q, &rs);
      scales[m] = s;
      if (rowsum) rowsum[m] = rs;
      if (bits == 8)
        memcpy((int8_t *)codes + m * K, q, (size_t)K);
      else
        hbo_pack_int4(q, 1, K, (uint32_t *)codes + m * (K / 8));
    }
    free(t);
    free(xr);
    free(q);
  }
  return 0;
}

/* Eq. 9 without the normalisation layer: with hadamard != 0 the row is
 * rotated first (X_r = Hadamard(X)); with hadamard == 0 it is quantised as
 * is (plain BitLinear input). */
int hbo_quantize(const void *x, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                 int hadamard, int bits, void *codes, float *scales,
                 int32_t *rowsum, float *xr_out) {
  return quantize_rows(x, x_dtype, M, K, ldx, 0, NULL, hadamard, bits, codes, scales, rowsum,
                       xr_out);
}

/* Eq. 9 with its normalisation layer: X_r = Hadamard(RMSNorm(X)) (or
 * RMSNorm(X) alone with hadamard == 0), then quantised. */
int hbo_norm_quantize(const void *x, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                      const float *gain, int hadamard, int bits, void *codes, float *scales,
                      int32_t *rowsum, float *xr_out) {
  return quantize_rows(x, x_dtype, M, K, ldx, 1, gain, hadamard, bits, codes, scales, rowsum,
                       xr_out);
}

/* ------------------------------------------------------------------ */
/* Backward of the rotation  [BNv2 §3.4 "Gradient Handling Through the */
/* Hadamard Transformation", Eq. 10]                                   */
/* ------------------------------------------------------------------ */

/* dX = H^T dY row by row, written out as the transposed matrix product
 * dx[k] = sum_j H[j][k] dy[j], with the entries of the normalised
 * Sylvester matrix in closed form: H[j][k] = (-1)^popcount(j & k) / sqrt(K).
 * O(K^2) per row on purpose: it does not use the fast transform, so it is
 * an independent check of the claim that the backward is the forward
 * transform again.  dx is fp64 [M][K]. */
int hbo_hadamard_backward(const void *dy, int dy_dtype, int64_t M, int64_t K, int64_t lddy,
                          double *dx) {
  if (!is_pow2(K) || lddy < K || M < 0) return 2;
  const double scale = 1.0 / sqrt((double)K);
#pragma omp parallel
  {
    double *g = (double *)malloc((size_t)K * sizeof(double));
#pragma omp for schedule(static)
    for (int64_t m = 0; m < M; m++) {
      for (int64_t j = 0; j < K; j++) g[j] = (double)load_elem(dy, dy_dtype, m * lddy + j);
      for (int64_t k = 0; k < K; k++) {
        double s = 0.0;
        for (int64_t j = 0; j < K; j++) {
          const double h = (__builtin_popcountll((unsigned long long)(j & k)) & 1) ? -1.0 : 1.0;
          s += h * g[j];
        }
        dx[m * K + k] = s * scale;
      }
    }
    free(g);
  }
  return 0;
}

/* ------------------------------------------------------------------ */
/* Ternary weight quantizer  [BNv2 §3.4 "Weight Quantization",         */
/* Eq. 1-2]                                                            */
/* ------------------------------------------------------------------ */

void hbo_pack_ternary(const int8_t *q, int64_t N, int64_t K, uint32_t *packed) {
  for (int64_t n = 0; n < N; n++)
    for (int64_t w = 0; w < K / 16; w++) {
      uint32_t word = 0;
      for (int j = 0; j < 16; j++) {
        int s = j / 4, b = j % 4;
        uint32_t c = (uint32_t)(q[n * K + 16 * w + j] + 1);
        word |= c << (8 * b + 2 * s);
      }
      packed[n * (K / 16) + w] = word;
    }
}

/* Returns the number of invalid 2-bit fields (value 3) met; they decode as 0. */
int64_t hbo_unpack_ternary(const uint32_t *packed, int64_t N, int64_t K, int8_t *q) {
  int64_t bad = 0;
  for (int64_t n = 0; n < N; n++)
    for (int64_t w = 0; w < K / 16; w++) {
      uint32_t word = packed[n * (K / 16) + w];
      for (int j = 0; j < 16; j++) {
        int s = j / 4, b = j % 4;
        int c = (int)((word >> (8 * b + 2 * s)) & 3u);
        if (c == 3) {
          bad++;
          c = 1;
        }
        q[n * K + 16 * w + j] = (int8_t)(c - 1);
      }
    }
  return bad;
}

/* alpha = mean(|W|) over the whole matrix (fp64 sum, one fp32 result);
 * q = RoundClip(W / (alpha + eps), -1, 1).  W is fp32 or bf16 [N][K].
 * Writes the packed codes, alpha, and (nullable) the int8 codes. */
int hbo_ternarize(const void *w, int w_dtype, int64_t N, int64_t K,
                  uint32_t *packed, float *alpha, int8_t *q_out) {
  if (N <= 0 || K <= 0 || K % 16 != 0) return 2;
  double sum = 0.0;
  for (int64_t i = 0; i < N * K; i++) sum += fabs((double)load_elem(w, w_dtype, i));
  float a = (float)(sum / ((double)N * (double)K));
  float d = a + HBO_EPS;
  int8_t *q = (int8_t *)malloc((size_t)(N * K));
  for (int64_t i = 0; i < N * K; i++)
    q[i] = (int8_t)round_clip(load_elem(w, w_dtype, i) / d, -1.0f, 1.0f);
  hbo_pack_ternary(q, N, K, packed);
  if (q_out) memcpy(q_out, q, (size_t)(N * K));
  free(q);
  *alpha = a;
  return 0;
}

/* Weight and activation rotation  [BNv2 §3.4 "Ablation Study: Why
 * Activation-Only Hadamard Transformation", Table 5]: the ternarised matrix
 * is Q_w(W H^T).  Row n of W H^T is H applied to row n of W (H is
 * symmetric); each row is rotated in fp64 (the transform of Eq. 3-6),
 * rounded once to fp32, and the fp32 matrix is ternarised as by
 * hbo_ternarize.  wr_out (nullable) receives that fp32 matrix [N][K]. */
int hbo_ternarize_rotated(const void *w, int w_dtype, int64_t N, int64_t K, uint32_t *packed,
                          float *alpha, int8_t *q_out, float *wr_out) {
  if (N <= 0 || K < 16 || !is_pow2(K)) return 2;
  double *y = (double *)malloc((size_t)(N * K) * sizeof(double));
  float *wr = (float *)malloc((size_t)(N * K) * sizeof(float));
  int rc = hbo_hadamard(w, w_dtype, N, K, K, y);
  if (rc == 0) {
    for (int64_t i = 0; i < N * K; i++) wr[i] = (float)y[i];
    rc = hbo_ternarize(wr, HBO_F32, N, K, packed, alpha, q_out);
    if (rc == 0 && wr_out) memcpy(wr_out, wr, (size_t)(N * K) * sizeof(float));
  }
  free(y);
  free(wr);
  return rc;
}

/* ------------------------------------------------------------------ */
/* Integer matmul and the full layer  [BNv2 §3.4 "H-BitLinear", Eq. 9] */
/* ------------------------------------------------------------------ */

static int8_t code_at(const void *codes, int bits, int64_t K, int64_t m, int64_t k) {
  if (bits == 8) return ((const int8_t *)codes)[m * K + k];
  uint32_t word = ((const uint32_t *)codes)[m * (K / 8) + k / 8];
  int j = (int)(k % 8), h = j / 4, b = j % 4;
  int nib = (int)((word >> (8 * b + 4 * h)) & 0xfu);
  return (int8_t)(nib >= 8 ? nib - 16 : nib);
}

static int8_t weight_at(const uint32_t *packed, int64_t K, int64_t n, int64_t k) {
  uint32_t word = packed[n * (K / 16) + k / 16];
  int j = (int)(k % 16), s = j / 4, b = j % 4;
  int c = (int)((word >> (8 * b + 2 * s)) & 3u);
  return (int8_t)(c - 1);
}

/* acc[m][n] = sum_k qx[m][k] * qw[n][k]: a plain triple loop.
 * Returns 0, 2 on a bad shape, 3 if a sum does not fit int32 (cannot happen
 * for K <= 2^23). */
int hbo_gemm_i32(const void *codes, int bits, const uint32_t *packed, int64_t M,
                 int64_t N, int64_t K, int32_t *acc) {
  if (M < 0 || N <= 0 || K <= 0 || K % 16 != 0 || (bits != 8 && bits != 4)) return 2;
  int overflow = 0;
#pragma omp parallel for schedule(static) reduction(| : overflow)
  for (int64_t m = 0; m < M; m++) {
    for (int64_t n = 0; n < N; n++) {
      int64_t s = 0;
      for (int64_t k = 0; k < K; k++)
        s += (int64_t)code_at(codes, bits, K, m, k) * (int64_t)weight_at(packed, K, n, k);
      if (s > INT32_MAX || s < INT32_MIN) overflow = 1;
      acc[m * N + n] = (int32_t)s;
    }
  }
  return overflow ? 3 : 0;
}

/* Y = Q_w(W) . Q(X_r), row-major: y[m][n] = (s_m * alpha) * acc[m][n].
 * y64 (fp64) is the value; y_bf16 (nullable) is the same value rounded to
 * bf16 through fp32, the output type of the GPU layer. */
int hbo_dequant_output(const int32_t *acc, const float *scales, float alpha,
                       int64_t M, int64_t N, double *y64, uint16_t *y_bf16) {
  for (int64_t m = 0; m < M; m++)
    for (int64_t n = 0; n < N; n++) {
      double v = (double)scales[m] * (double)alpha * (double)acc[m * N + n];
      if (y64) y64[m * N + n] = v;
      if (y_bf16) y_bf16[m * N + n] = hbo_f32_to_bf16((float)v);
    }
  return 0;
}

/* The whole forward for one layer: quantise X (optionally rotating it),
 * integer matmul against packed ternary weights, rescale.  Writes y64
 * [M][N]; the codes/scales/acc scratch is allocated here. */
int hbo_forward(const void *x, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                int hadamard, int bits, const uint32_t *packed, float alpha,
                int64_t N, double *y64) {
  size_t code_bytes = (bits == 8) ? (size_t)(M * K) : (size_t)(M * (K / 8)) * 4;
  void *codes = malloc(code_bytes ? code_bytes : 1);
  float *scales = (float *)malloc((size_t)(M > 0 ? M : 1) * sizeof(float));
  int32_t *acc = (int32_t *)malloc((size_t)(M * N > 0 ? M * N : 1) * sizeof(int32_t));
  int rc = hbo_quantize(x, x_dtype, M, K, ldx, hadamard, bits, codes, scales, NULL, NULL);
  if (rc == 0) rc = hbo_gemm_i32(codes, bits, packed, M, N, K, acc);
  if (rc == 0) rc = hbo_dequant_output(acc, scales, alpha, M, N, y64, NULL);
  free(codes);
  free(scales);
  free(acc);
  return rc;
}

/* ------------------------------------------------------------------ */
/* Post-RoPE QKV / KV-cache quantiser  [BNv2 §3.4 "QKV Attention       */
/* Quantization: Post-RoPE INT4/3-bit"]                                 */
/* ------------------------------------------------------------------ */

/* Reading (the pages say "unsigned integers using the absmax function" and
 * describe the unsigned range as the signed one shifted): each group of D
 * elements (one head of one token) is quantised with the absmax quantiser
 * of Eq. 7 at b bits, Q = 2^(b-1) - 1:
 *   gamma = max |x|,  v = RoundClip(x * Q / (gamma + eps), -2^(b-1), 2^(b-1) - 1),
 *   u = v + 2^(b-1) in [0, 2^b - 1],   scale = gamma / Q,
 * so x ~ (u - 2^(b-1)) * scale.  The factor Q/(gamma+eps) is one fp32 value
 * per group, as in Eq. 7.
 * Packing (bit-exact contract with the library): b = 8 one byte per code;
 * b = 4 two codes per byte, code 2i in the low nibble; b = 3 eight codes per
 * three bytes, code j of the group of 8 at bits [3j, 3j + 3) of the 24-bit
 * little-endian value.  A group of D codes takes D * b / 8 bytes. */
static void kv_quant_group(const void *x, int x_dtype, int64_t off, int64_t D, int bits,
                           uint8_t *codes, float *scale) {
  float gamma = 0.0f;
  for (int64_t k = 0; k < D; k++) {
    float a = fabsf(load_elem(x, x_dtype, off + k));
    if (a > gamma) gamma = a;
  }
  const int half = 1 << (bits - 1);
  const float q = (float)(half - 1);
  const float f = q / (gamma + HBO_EPS);
  *scale = gamma / q;
  memset(codes, 0, (size_t)(D * bits / 8));
  for (int64_t k = 0; k < D; k++) {
    const float v = round_clip(load_elem(x, x_dtype, off + k) * f, (float)-half, (float)(half - 1));
    const unsigned u = (unsigned)((int)v + half);
    if (bits == 8) {
      codes[k] = (uint8_t)u;
    } else if (bits == 4) {
      codes[k / 2] |= (uint8_t)(u << (4 * (k % 2)));
    } else {
      const int64_t g = k / 8, j = k % 8, bit = 24 * g + 3 * j;
      for (int t = 0; t < 3; t++)
        if ((u >> t) & 1u) codes[(bit + t) / 8] |= (uint8_t)(1u << ((bit + t) % 8));
    }
  }
}

/* x: [B][S][H][D] (fp32 or bf16), contiguous.  codes: [B][S][H][D*bits/8]
 * bytes, scales: [B][S][H].  With keep_bos8, position 0 of every sequence
 * (the [BOS] token, whose KV heads the pages keep at 8 bits) is also
 * quantised at 8 bits into bos_codes [B][H][D] and bos_scales [B][H].
 * Returns 0, or 2 for a bad shape / mode. */
int hbo_kv_quant(const void *x, int x_dtype, int64_t B, int64_t S, int64_t H, int64_t D, int bits,
                 int keep_bos8, uint8_t *codes, float *scales, uint8_t *bos_codes, float *bos_scales) {
  if (B < 0 || S < 1 || H < 1 || D < 8 || D % 8 != 0) return 2;
  if (bits != 3 && bits != 4 && bits != 8) return 2;
  const int64_t cb = D * bits / 8;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < B * S; t++) {
    for (int64_t h = 0; h < H; h++) {
      const int64_t g = t * H + h;
      kv_quant_group(x, x_dtype, g * D, D, bits, codes + g * cb, scales + g);
      if (keep_bos8 && t % S == 0) {
        const int64_t b = t / S;
        kv_quant_group(x, x_dtype, g * D, D, 8, bos_codes + (b * H + h) * D, bos_scales + b * H + h);
      }
    }
  }
  return 0;
}

/* Inverse of the packing and the shift: x_hat = (u - 2^(b-1)) * scale, fp64
 * [G][D] for G groups. */
int hbo_kv_dequant(const uint8_t *codes, const float *scales, int64_t G, int64_t D, int bits, double *x_hat) {
  if (G < 0 || D < 8 || D % 8 != 0 || (bits != 3 && bits != 4 && bits != 8)) return 2;
  const int64_t cb = D * bits / 8;
  const int half = 1 << (bits - 1);
  for (int64_t g = 0; g < G; g++) {
    const uint8_t *c = codes + g * cb;
    for (int64_t k = 0; k < D; k++) {
      unsigned u;
      if (bits == 8) {
        u = c[k];
      } else if (bits == 4) {
        u = (c[k / 2] >> (4 * (k % 2))) & 15u;
      } else {
        const int64_t bit = 24 * (k / 8) + 3 * (k % 8);
        u = 0;
        for (int t = 0; t < 3; t++) u |= (unsigned)((c[(bit + t) / 8] >> ((bit + t) % 8)) & 1u) << t;
      }
      x_hat[g * D + k] = ((double)u - half) * (double)scales[g];
    }
  }
  return 0;
}

/* Number of OpenMP threads the parallel loops above use (1 without OpenMP). */
int hbo_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Sets the number of OpenMP threads of the calling thread's later parallel
 * loops (used to time the oracle at one thread and at all cores). */
void hbo_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}
