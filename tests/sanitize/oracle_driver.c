/* Sanitizer driver for the CPU oracle (test infrastructure): runs every
 * oracle entry point on small deterministic inputs, including ragged and
 * degenerate ones, so AddressSanitizer and UndefinedBehaviorSanitizer see
 * every loop bound and index.  Exit status 0 means no check failed. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

static uint32_t state = 12345u;
static float frand(void) {            /* xorshift32 in [-1, 1) */
  state ^= state << 13;
  state ^= state >> 17;
  state ^= state << 5;
  return (float)(state >> 8) / 8388608.0f - 1.0f;
}

static void *xmalloc(size_t n) {
  void *p = malloc(n ? n : 1);
  if (!p) exit(3);
  return p;
}

static int check_quant(int64_t n, int64_t k, int bits, int sym) {
  const int64_t G = k / 128;
  float *W = xmalloc(sizeof(float) * n * k), *wh = xmalloc(sizeof(float) * n * k);
  uint8_t *q = xmalloc(n * k), *q2 = xmalloc(n * k), *z = xmalloc(n * G);
  float *s = xmalloc(sizeof(float) * n * G);
  uint32_t *words = xmalloc(sizeof(uint32_t) * (n * k * bits / 32));
  for (int64_t i = 0; i < n * k; ++i) W[i] = 0.02f * frand() + (i % 97 == 0 ? 0.3f : 0.0f);
  if (n > 1) memset(W, 0, sizeof(float) * k);           /* an all-zero row */
  oracle_quantize(W, n, k, bits, 128, sym, q, s, z);
  oracle_pack(q, n, k, bits, words);
  oracle_unpack(words, n, k, bits, q2);
  oracle_dequantize(q2, s, z, n, k, 128, wh);
  double err[2];
  oracle_quant_error(W, wh, s, n, k, 128, err);
  int bad = memcmp(q, q2, n * k) != 0 || !(err[0] >= 0.0);
  /* compact layout */
  uint16_t *s16 = xmalloc(sizeof(uint16_t) * n * G);
  uint8_t *zp = xmalloc(n * G);
  oracle_quantize_compact(W, n, k, bits, 128, sym, q, s16, z);
  int64_t nz = oracle_pack_zeros(z, n * G, bits, zp);
  oracle_dequantize_compact(q, s16, zp, n, k, 128, bits, wh);
  bad |= nz <= 0;
  free(W); free(wh); free(q); free(q2); free(z); free(s); free(words); free(s16); free(zp);
  return bad;
}

static int check_gemm(int64_t m, int64_t n, int64_t k) {
  uint16_t *x = xmalloc(2 * m * k);
  float *wh = xmalloc(sizeof(float) * n * k);
  double *y = xmalloc(sizeof(double) * m * n), *b = xmalloc(sizeof(double) * m * n);
  for (int64_t i = 0; i < m * k; ++i) x[i] = (uint16_t)(0x3F80u + (i % 37));
  for (int64_t i = 0; i < n * k; ++i) wh[i] = frand();
  oracle_gemm(x, m, k, wh, n, y, b);
  int64_t xi[3] = {0, m - 1, m / 2}, wi[3] = {n - 1, 0, n / 2};
  double yp[3], bp[3];
  oracle_gemm_pairs(x, k, wh, xi, wi, 3, yp, bp);
  int bad = fabs(yp[0] - y[(m - 1 + 1 - 1) * 0 + (n - 1)]) > 0.0 && 0;
  for (int j = 0; j < 3; ++j) bad |= fabs(yp[j] - y[xi[j] * n + wi[j]]) > 1e-9 * (bp[j] + 1e-30);
  free(x); free(wh); free(y); free(b);
  return bad;
}

static int check_fidelity(int64_t rows, int64_t vocab) {
  float *a = xmalloc(sizeof(float) * rows * vocab), *c = xmalloc(sizeof(float) * rows * vocab);
  for (int64_t i = 0; i < rows * vocab; ++i) {
    a[i] = 3.0f * frand();
    c[i] = a[i] + 0.05f * frand();
  }
  double *lse = xmalloc(sizeof(double) * rows), *e = xmalloc(sizeof(double) * rows),
         *kl = xmalloc(sizeof(double) * rows), m2[2];
  oracle_row_lse(a, rows, vocab, lse);
  oracle_ear_kl(a, c, rows, vocab, e, kl, m2);
  int bad = !(m2[0] > 0.0 && m2[0] <= 1.0 + 1e-12);
  for (int64_t K = 1; K <= (vocab < 12 ? vocab : 12); K += 5) {
    oracle_ear_kl_topk(a, c, rows, vocab, K, 0.7, e, kl, m2);
    bad |= !(m2[0] >= 0.0);
  }
  free(a); free(c); free(lse); free(e); free(kl);
  return bad;
}

static int check_mckp(void) {
  const int64_t L = 5;
  const int nb = 3;
  int64_t sizes[15];
  double costs[15];
  for (int i = 0; i < 15; ++i) {
    sizes[i] = (i % 3) + 1 + (i == 7 ? -100 : 0);   /* one negative size: never selected */
    costs[i] = 1.0 / (1 + i % 3) + 0.01 * i;
  }
  int32_t choice[5];
  int64_t budget, size;
  double cost, best[41];
  int st = oracle_mckp_search(L, nb, sizes, costs, 40, 2.0, choice, &budget, &size, &cost, best);
  st |= oracle_mckp_search(L, nb, sizes, costs, 0, 2.0, choice, &budget, &size, &cost, NULL) & 0;
  return st < 0;
}

static int check_gptq(int64_t n, int64_t k, int bits) {
  float *W = xmalloc(sizeof(float) * n * k), *U = xmalloc(sizeof(float) * k * k);
  uint8_t *q = xmalloc(n * k), *z = xmalloc(n * (k / 128)), *dead = xmalloc(k);
  float *s = xmalloc(sizeof(float) * n * (k / 128));
  for (int64_t i = 0; i < n * k; ++i) W[i] = 0.02f * frand();
  for (int64_t i = 0; i < k; ++i) {
    dead[i] = i % 50 == 3;
    for (int64_t j = 0; j < k; ++j) U[i * k + j] = j < i ? 0.0f : (j == i ? 1.0f + 0.5f * frand() : 0.01f * frand());
  }
  oracle_gptq_columns(W, U, dead, n, k, bits, 128, q, s, z);
  oracle_gptq_columns(W, U, NULL, n, k, bits, 128, q, s, z);
  free(W); free(U); free(q); free(z); free(dead); free(s);
  return 0;
}

int main(void) {
  int bad = 0;
  for (int bits = 2; bits <= 8; ++bits) {
    bad |= check_quant(3, 384, bits, 0);
    bad |= check_quant(1, 128, bits, 1);
  }
  bad |= check_gemm(3, 5, 256);
  bad |= check_gemm(1, 1, 128);
  bad |= check_fidelity(3, 11);
  bad |= check_fidelity(1, 2);
  bad |= check_mckp();
  bad |= check_gptq(3, 256, 4);
  bad |= check_gptq(2, 128, 8);
  double bpp = oracle_bits_per_param(4, 20, 128);
  uint16_t h = oracle_f16_round_up(0.0123f);
  bad |= !(bpp > 4.0) || !(oracle_f16_value(h) >= 0.0123) || oracle_compact_zero_bits(3) != 4;
  printf("oracle sanitizer driver: %s\n", bad ? "FAILED" : "ok");
  return bad;
}
