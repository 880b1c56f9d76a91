/* Runs the C oracle on small cases, for a build with address and
 * undefined-behaviour sanitizers (and OpenMP).  Checks facts the definition
 * of softmax attention fixes, so a sanitized run also exercises the oracle's
 * indexing in both layouts and both element formats:
 *   - N = 1 gives O = V exactly;
 *   - every row of P sums to 1;
 *   - the 4-token closed form (O[1][0] = 2.492652734586...);
 *   - the row entry point agrees with the full forward, and rejects
 *     triples out of range.
 * Prints "ok <n>" on success, else the first failure, and exits non-zero. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_attention_fmt(const uint16_t* qkv_or_q, const uint16_t* k, const uint16_t* v, int layout,
                         int fmt, int B, int H, int N, int D, double scale, double* out, double* probs);
int oracle_attention_rows_fmt(const uint16_t* qkv_or_q, const uint16_t* k, const uint16_t* v,
                              int layout, int fmt, int B, int H, int N, int D, double scale,
                              const int64_t* rows, int64_t R, double* out);

static uint16_t bf16_of(float f) { /* exact for the small integers and halves used here */
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

static uint32_t rng_state = 12345u;
/* A value m / 64 with -128 <= m < 128, exact in both formats: its bits in
 * format fmt, and the value itself in *val. */
static uint16_t rand_bits(int fmt, float* val) {
  rng_state = rng_state * 1664525u + 1013904223u;
  const int m = (int)(rng_state >> 24) - 128;
  *val = (float)m / 64.0f;
  if (fmt == 1) { /* IEEE binary16: sign, 5-bit exponent (bias 15), 10-bit fraction */
    const float f = (float)m / 64.0f;
    if (m == 0) return 0;
    int e = 0;
    float a = fabsf(f);
    while (a >= 2.0f) { a /= 2.0f; ++e; }
    while (a < 1.0f) { a *= 2.0f; --e; }
    const unsigned mant = (unsigned)((a - 1.0f) * 1024.0f);
    return (uint16_t)((f < 0 ? 0x8000u : 0u) | ((unsigned)(e + 15) << 10) | mant);
  }
  return bf16_of((float)m / 64.0f);
}

static int fail(const char* what) {
  printf("FAIL %s\n", what);
  return 1;
}

int main(void) {
  int checks = 0;
  for (int fmt = 0; fmt < 2; ++fmt)
    for (int layout = 0; layout < 2; ++layout)
      for (int D = 1; D <= 72; D += 71) {
        const int B = 2, H = 3, N = 37;
        const size_t n = (size_t)B * H * N * D;
        uint16_t* qkv = malloc(3 * n * sizeof(uint16_t));
        float* val = malloc(3 * n * sizeof(float));
        double* out = malloc(n * sizeof(double));
        double* probs = malloc((size_t)B * H * N * N * sizeof(double));
        for (size_t i = 0; i < 3 * n; ++i) qkv[i] = rand_bits(fmt, &val[i]);
        const uint16_t* q = qkv;
        const uint16_t* k = layout == 0 ? qkv + n : NULL;
        const uint16_t* v = layout == 0 ? qkv + 2 * n : NULL;
        if (oracle_attention_fmt(q, k, v, layout, fmt, B, H, N, D, 0.3, out, probs) != 0)
          return fail("forward status");
        for (int r = 0; r < B * H * N; ++r) {
          double s = 0.0;
          for (int j = 0; j < N; ++j) s += probs[(size_t)r * N + j];
          if (fabs(s - 1.0) > 1e-12) return fail("row of P does not sum to 1");
          ++checks;
        }
        int64_t rows[3 * 4] = {0, 0, 0, 1, 2, 36, 1, 0, 17, 0, 2, 5};
        double ro[4 * 72];
        if (oracle_attention_rows_fmt(q, k, v, layout, fmt, B, H, N, D, 0.3, rows, 4, ro) != 0)
          return fail("rows status");
        for (int r = 0; r < 4; ++r)
          for (int d = 0; d < D; ++d) {
            const int64_t b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
            if (ro[r * D + d] != out[((b * N + i) * H + h) * D + d]) return fail("rows vs forward");
            ++checks;
          }
        int64_t bad[3] = {0, 3, 0}; /* head 3 of 3 */
        if (oracle_attention_rows_fmt(q, k, v, layout, fmt, B, H, N, D, 0.3, bad, 1, ro) != -5)
          return fail("row out of range accepted");
        /* N = 1: O = V exactly (V of token 0 starts at element 2 D when
         * packed, at element 2 n in the separate layout) */
        if (oracle_attention_fmt(q, k, v, layout, fmt, 1, 1, 1, D, 0.3, out, NULL) != 0)
          return fail("N = 1 status");
        for (int d = 0; d < D; ++d) {
          if (out[d] != (double)val[(layout == 1 ? 2 * (size_t)D : 2 * n) + d]) return fail("N = 1 gives V");
          ++checks;
        }
        free(val);
        free(qkv);
        free(out);
        free(probs);
      }
  /* the 4-token case: Q[i][0] = i, K[l][0] = 8 l, V[l][0] = l, scale 1/8 */
  {
    uint16_t qkv[4 * 3 * 64];
    memset(qkv, 0, sizeof qkv);
    for (int t = 0; t < 4; ++t) {
      qkv[(t * 3 + 0) * 64] = bf16_of((float)t);
      qkv[(t * 3 + 1) * 64] = bf16_of(8.0f * t);
      qkv[(t * 3 + 2) * 64] = bf16_of((float)t);
    }
    double o[4 * 64];
    if (oracle_attention_fmt(qkv, NULL, NULL, 1, 0, 1, 1, 4, 64, 0.125, o, NULL) != 0)
      return fail("4-token status");
    const double e = exp(1.0);
    const double want = (e + 2 * e * e + 3 * e * e * e) / (1 + e + e * e + e * e * e);
    if (fabs(o[64] - want) > 1e-12 || fabs(o[0] - 1.5) > 1e-12) return fail("4-token closed form");
    ++checks;
  }
  printf("ok %d\n", checks);
  return 0;
}
