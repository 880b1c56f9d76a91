/*
 * Reference (oracle) for the bidirectional multi-head self-attention forward
 * of a ViT / SigLIP vision encoder.  TEST INFRASTRUCTURE ONLY: the tests, the
 * smoke check and the benchmark's CPU-baseline leg use it; the library's
 * product path never links, loads or calls it.
 *
 * What it computes.  The Pi0 Flash Attention tutorial (section 1) states that
 * swapping the encoder's attention for Flash Attention leaves the model and
 * its output quality unchanged, and its section 4.2 table shows the same
 * accuracy before and after; so the fast path must reach the plain
 * definition of softmax attention, and this file is that definition written
 * out, with no tiling, fusion or reordering:
 *
 *   for every image b and head h, with Q, K, V the N x D inputs of (b, h)
 *   (bf16 or fp16) widened exactly to double:
 *     S[i][j] = scale * sum_d Q[i][d] * K[j][d]
 *     P[i][j] = exp(S[i][j] - max_j' S[i][j']) / sum_j'' exp(S[i][j''] - max_j' S[i][j'])
 *     O[i][d] = sum_j P[i][j] * V[j][d]
 *
 * Subtracting the row maximum leaves P unchanged mathematically and keeps
 * exp() finite in double.  All tokens attend to all tokens (no mask) and no
 * dropout is applied: the encoder is bidirectional and runs in inference.
 *
 * Input layouts (the tutorial's section 3.2 feeds the attention from the
 * block's fused qkv projection):
 *   layout 0, separate: q, k, v each [B][H][N][D]
 *   layout 1, packed:   one buffer [B][N][3][H][D] (slot 0 = Q, 1 = K, 2 = V);
 *                       k and v are ignored
 * Output: double, always in logical order [B][N][H][D].
 *
 * Element formats: bf16 (fmt 0) or IEEE 754 binary16, fp16 (fmt 1); either is
 * widened exactly to double.
 * Precision: fp64 throughout.
 * Parallelism: OpenMP over (b, h) pairs, static schedule.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Exact widening of a bfloat16 bit pattern: the top 16 bits of a float. */
static double bf16_to_double(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* Exact widening of an IEEE 754 binary16 bit pattern: 1 sign bit, 5
 * exponent bits (bias 15), 10 fraction bits; exponent 0 holds zero and the
 * subnormals fraction * 2^-24, exponent 31 infinity and NaN. */
static double f16_to_double(uint16_t bits) {
  const int sign = bits >> 15, e = (bits >> 10) & 31, f = bits & 1023;
  double mag;
  if (e == 0) mag = ldexp((double)f, -24);
  else if (e == 31) mag = f ? NAN : INFINITY;
  else mag = ldexp(1024.0 + f, e - 25);  /* (1 + f/1024) * 2^(e-15) */
  return sign ? -mag : mag;
}

static double widen(uint16_t bits, int fmt) {
  return fmt == 1 ? f16_to_double(bits) : bf16_to_double(bits);
}

/* Offset, in elements, of element (b, n, h, d) of tensor `which`
 * (0 = Q, 1 = K, 2 = V) in the given layout. */
static int64_t elem_offset(int layout, int which, int64_t B, int64_t H, int64_t N,
                           int64_t D, int64_t b, int64_t n, int64_t h, int64_t d) {
  (void)B;
  if (layout == 1) return (((b * N + n) * 3 + which) * H + h) * D + d;
  return ((b * H + h) * N + n) * D + d;
}

static const uint16_t* tensor_base(int layout, int which, const uint16_t* qkv_or_q,
                                   const uint16_t* k, const uint16_t* v) {
  if (layout == 1) return qkv_or_q;
  return which == 0 ? qkv_or_q : (which == 1 ? k : v);
}

/* Gathers the N x D matrix of tensor `which` for (b, h) into dst (row-major). */
static void gather(double* dst, int layout, int fmt, int which, const uint16_t* qkv_or_q,
                   const uint16_t* k, const uint16_t* v, int64_t B, int64_t H,
                   int64_t N, int64_t D, int64_t b, int64_t h) {
  const uint16_t* base = tensor_base(layout, which, qkv_or_q, k, v);
  for (int64_t n = 0; n < N; ++n)
    for (int64_t d = 0; d < D; ++d)
      dst[n * D + d] = widen(base[elem_offset(layout, which, B, H, N, D, b, n, h, d)], fmt);
}

/* One query row of one (b, h): q_row[D] is Q_i; fills p_row[N] with P[i][:]
 * and o_row[D] with O[i][:].  K and V are the gathered N x D matrices. */
static void attend_row(const double* q_row, const double* K, const double* V, int64_t N,
                       int64_t D, double scale, double* p_row, double* o_row) {
  /* S[i][j] = scale * <Q_i, K_j> */
  for (int64_t j = 0; j < N; ++j) {
    double dot = 0.0;
    for (int64_t d = 0; d < D; ++d) dot += q_row[d] * K[j * D + d];
    p_row[j] = scale * dot;
  }
  /* softmax over the key axis */
  double m = p_row[0];
  for (int64_t j = 1; j < N; ++j)
    if (p_row[j] > m) m = p_row[j];
  double l = 0.0;
  for (int64_t j = 0; j < N; ++j) {
    p_row[j] = exp(p_row[j] - m);
    l += p_row[j];
  }
  for (int64_t j = 0; j < N; ++j) p_row[j] /= l;
  /* O[i][:] = sum_j P[i][j] V[j][:] */
  for (int64_t d = 0; d < D; ++d) o_row[d] = 0.0;
  for (int64_t j = 0; j < N; ++j)
    for (int64_t d = 0; d < D; ++d) o_row[d] += p_row[j] * V[j * D + d];
}

static int check_args(const uint16_t* qkv_or_q, const uint16_t* k, const uint16_t* v,
                      int layout, int fmt, int B, int H, int N, int D) {
  if (!qkv_or_q) return -1;
  if (fmt != 0 && fmt != 1) return -2;
  if (layout != 0 && layout != 1) return -2;
  if (layout == 0 && (!k || !v)) return -1;
  if (B < 0 || H < 0 || N < 0 || D < 1) return -3;
  return 0;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/*
 * Full forward.  fmt: 0 = bf16 inputs, 1 = fp16.  out: [B][N][H][D] doubles.
 * probs: NULL, or [B][H][N][N] doubles receiving P.  Returns 0, or a
 * negative value on a bad argument (-1 missing pointer, -2 bad layout or
 * format, -3 bad size, -4 out of memory).
 */
int oracle_attention_fmt(const uint16_t* qkv_or_q, const uint16_t* k, const uint16_t* v,
                         int layout, int fmt, int B, int H, int N, int D, double scale,
                         double* out, double* probs) {
  int rc = check_args(qkv_or_q, k, v, layout, fmt, B, H, N, D);
  if (rc) return rc;
  if (!out) return -1;
  if (B == 0 || H == 0 || N == 0) return 0;
  int64_t pairs = (int64_t)B * H;
  int failed = 0;
#pragma omp parallel
  {
    double* Q = malloc(sizeof(double) * (size_t)N * D);
    double* K = malloc(sizeof(double) * (size_t)N * D);
    double* V = malloc(sizeof(double) * (size_t)N * D);
    double* p = malloc(sizeof(double) * (size_t)N);
    double* o = malloc(sizeof(double) * (size_t)D);
    int ok = Q && K && V && p && o;
#pragma omp for schedule(static)
    for (int64_t bh = 0; bh < pairs; ++bh) {
      if (!ok) continue;
      int64_t b = bh / H, h = bh % H;
      gather(Q, layout, fmt, 0, qkv_or_q, k, v, B, H, N, D, b, h);
      gather(K, layout, fmt, 1, qkv_or_q, k, v, B, H, N, D, b, h);
      gather(V, layout, fmt, 2, qkv_or_q, k, v, B, H, N, D, b, h);
      for (int64_t i = 0; i < N; ++i) {
        attend_row(Q + i * D, K, V, N, D, scale, p, o);
        for (int64_t d = 0; d < D; ++d) out[((b * N + i) * H + h) * D + d] = o[d];
        if (probs)
          for (int64_t j = 0; j < N; ++j) probs[((b * H + h) * N + i) * N + j] = p[j];
      }
    }
    if (!ok) {
#pragma omp atomic write
      failed = 1;
    }
    free(Q); free(K); free(V); free(p); free(o);
  }
  return failed ? -4 : 0;
}

/* The full forward on bf16 inputs. */
int oracle_attention(const uint16_t* qkv_or_q, const uint16_t* k, const uint16_t* v,
                     int layout, int B, int H, int N, int D, double scale, double* out,
                     double* probs) {
  return oracle_attention_fmt(qkv_or_q, k, v, layout, 0, B, H, N, D, scale, out, probs);
}

/*
 * Selected rows only, for spot checks of large inputs.  rows: R triples
 * (b, h, i) as int64; out: [R][D] doubles with O[b][i][h][:].  Uses the same
 * per-row routine as oracle_attention_fmt().  Returns 0 or a negative error
 * (-5: a triple out of range).
 */
int oracle_attention_rows_fmt(const uint16_t* qkv_or_q, const uint16_t* k, const uint16_t* v,
                              int layout, int fmt, int B, int H, int N, int D, double scale,
                              const int64_t* rows, int64_t R, double* out) {
  int rc = check_args(qkv_or_q, k, v, layout, fmt, B, H, N, D);
  if (rc) return rc;
  if (R > 0 && (!rows || !out)) return -1;
  for (int64_t r = 0; r < R; ++r) {
    if (rows[3 * r] < 0 || rows[3 * r] >= B || rows[3 * r + 1] < 0 || rows[3 * r + 1] >= H ||
        rows[3 * r + 2] < 0 || rows[3 * r + 2] >= N)
      return -5;
  }
  int failed = 0;
#pragma omp parallel
  {
    double* Q = malloc(sizeof(double) * (size_t)D);
    double* K = malloc(sizeof(double) * (size_t)N * D);
    double* V = malloc(sizeof(double) * (size_t)N * D);
    double* p = malloc(sizeof(double) * (size_t)N);
    int ok = Q && K && V && p;
#pragma omp for schedule(dynamic, 4)
    for (int64_t r = 0; r < R; ++r) {
      if (!ok) continue;
      int64_t b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
      const uint16_t* qb = tensor_base(layout, 0, qkv_or_q, k, v);
      for (int64_t d = 0; d < D; ++d)
        Q[d] = widen(qb[elem_offset(layout, 0, B, H, N, D, b, i, h, d)], fmt);
      gather(K, layout, fmt, 1, qkv_or_q, k, v, B, H, N, D, b, h);
      gather(V, layout, fmt, 2, qkv_or_q, k, v, B, H, N, D, b, h);
      attend_row(Q, K, V, N, D, scale, p, out + r * D);
    }
    if (!ok) {
#pragma omp atomic write
      failed = 1;
    }
    free(Q); free(K); free(V); free(p);
  }
  return failed ? -4 : 0;
}

/* Selected rows on bf16 inputs. */
int oracle_attention_rows(const uint16_t* qkv_or_q, const uint16_t* k, const uint16_t* v,
                          int layout, int B, int H, int N, int D, double scale,
                          const int64_t* rows, int64_t R, double* out) {
  return oracle_attention_rows_fmt(qkv_or_q, k, v, layout, 0, B, H, N, D, scale, rows, R, out);
}

/* Exact widening of one 16-bit pattern (fmt 0 bf16, 1 fp16), for tests. */
double oracle_widen(unsigned bits, int fmt) { return widen((uint16_t)bits, fmt); }
