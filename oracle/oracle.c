/*
 * SLQ CPU oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct reference for what the SLQ hot path
 * computes.  Only the test suite, the smoke check and the bench's CPU-baseline
 * leg may load this library; the product path never does.  It shares no
 * source, header, table or helper with the HIP library.
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off -fopenmp (IEEE fp32 on SSE,
 * no contraction, round-to-nearest-even), see oracle/build.py.
 *
 * Sources (page title -> section):
 *  [SLQ-gist]   "Statistically-Lossless Quantization of Large Language Models"
 *               (gist.science technical summary): Methodology 1 (centering
 *               inefficiency gamma = 2M/R, the gamma-squared variance law),
 *               Methodology 2 (EAR as the summed min of the two next-token
 *               distributions, averaged over positions), Methodology 3
 *               (asymmetric integer group quantization, group size 128).
 *  [SLQ-readme] "SLQ" code README: Pipeline paragraph (asymmetric INT, g128,
 *               bit-widths 2..8), Usage 4 (weights packed to their per-layer
 *               bit-widths on load), Evaluation (EAR and KL of a model against
 *               its base).
 *  [SLQ-blog-en] "SLQ: Bridging the Gap ..." : The Motivation (next-token
 *               probability distribution), The Math of Asymmetry.
 *  [SLQ-readme] Search: the bit-width map adds 0.156 bits per parameter of
 *               scale and zero point (20 bits per 128-group); Evaluation:
 *               Uniform-4 at 4.16 bpp.
 *  [SLQ-summary] gist.science summary, "3. The SLQ Pipeline": bit-width
 *               allocation as a multiple-choice knapsack problem solved exactly
 *               (ILP) under a bit budget; [SLQ-readme] Pipeline paragraph: the
 *               budget is found by bisection until the target is met.
 * Where the pages leave a step open, the reading taken is stated at the
 * function (readings R1..R12 in the design notes).
 *
 * Parity pins: every function here is pinned by tests/test_oracle_*.py
 * against closed forms, brute force, worked values from the pages and
 * invariants; none is "parity unpinned".
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#include "oracle.h"

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Threads the parallel loops use from now on (the CPU baseline is timed on
 * one thread and on all). */
void oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* Round-to-nearest-even, then clamp to [0, maxq], all in fp32 (R4/R5). */
static float clamp_code(float v, int maxq) {
  if (v < 0.0f) return 0.0f;
  if (v > (float)maxq) return (float)maxq;
  return v;
}

/*
 * Asymmetric integer group quantization ([SLQ-gist] Methodology 3;
 * [SLQ-readme] Pipeline).  For each row n and each group g of `group`
 * consecutive inputs k:
 *   lo = min(0, min w), hi = max(0, max w)                (R1: 0 in range)
 *   s  = fl32(fl32(hi - lo) / (2^b - 1))                  (R3: fp32 divide)
 *   if s == 0 (all-zero group): s = 1, z = 0              (R2)
 *   z  = clamp(rint(fl32(-lo / s)), 0, 2^b - 1)           (R4)
 *   q  = clamp(rint(fl32(w / s)) + z, 0, 2^b - 1)         (R5)
 * Symmetric grid (comparison only, [SLQ-gist] Methodology 1):
 *   M = max |w|, s = fl32(2M / (2^b - 1)), z = 2^(b-1)    (R6)
 */
void oracle_quantize(const float *W, int64_t n, int64_t k, int bits, int group,
                     int symmetric, uint8_t *q, float *scales, uint8_t *zeros) {
  const int maxq = (1 << bits) - 1;
  const int64_t G = k / group;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n; ++r) {
    for (int64_t g = 0; g < G; ++g) {
      const float *w = W + r * k + g * group;
      float s;
      int z;
      if (!symmetric) {
        float lo = 0.0f, hi = 0.0f;
        for (int i = 0; i < group; ++i) {
          if (w[i] < lo) lo = w[i];
          if (w[i] > hi) hi = w[i];
        }
        float range = hi - lo;
        s = range / (float)maxq;
        if (s == 0.0f) {
          s = 1.0f;
          z = 0;
        } else {
          float zf = rintf((-lo) / s);
          z = (int)clamp_code(zf, maxq);
        }
      } else {
        float m = 0.0f;
        for (int i = 0; i < group; ++i) {
          float a = fabsf(w[i]);
          if (a > m) m = a;
        }
        float two_m = 2.0f * m;
        s = two_m / (float)maxq;
        if (s == 0.0f) s = 1.0f;
        z = 1 << (bits - 1);
      }
      scales[r * G + g] = s;
      zeros[r * G + g] = (uint8_t)z;
      for (int i = 0; i < group; ++i) {
        float t = rintf(w[i] / s);
        float v = clamp_code(t + (float)z, maxq);
        q[r * k + g * group + i] = (uint8_t)(int)v;
      }
    }
  }
}

/*
 * Dense bit-packing ([SLQ-readme] Usage 4: weights packed to their per-layer
 * bit-width).  R7: each row is one little-endian bitstream with no padding:
 * code j of the row occupies bits [j*b, j*b + b) of the integer
 * sum_i word_i * 2^(32 i).  A row of k codes fills k*b/32 words.
 */
void oracle_pack(const uint8_t *q, int64_t n, int64_t k, int bits, uint32_t *words) {
  const int64_t wpr = k * bits / 32;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n; ++r) {
    uint32_t *out = words + r * wpr;
    for (int64_t i = 0; i < wpr; ++i) out[i] = 0u;
    for (int64_t j = 0; j < k; ++j) {
      uint32_t code = q[r * k + j];
      for (int t = 0; t < bits; ++t) {
        int64_t bit = j * bits + t;
        if ((code >> t) & 1u) out[bit / 32] |= (1u << (bit % 32));
      }
    }
  }
}

void oracle_unpack(const uint32_t *words, int64_t n, int64_t k, int bits, uint8_t *q) {
  const int64_t wpr = k * bits / 32;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n; ++r) {
    const uint32_t *in = words + r * wpr;
    for (int64_t j = 0; j < k; ++j) {
      uint32_t code = 0;
      for (int t = 0; t < bits; ++t) {
        int64_t bit = j * bits + t;
        code |= ((in[bit / 32] >> (bit % 32)) & 1u) << t;
      }
      q[r * k + j] = (uint8_t)code;
    }
  }
}

/* Reconstruction w_hat = fl32((q - z) * s) of every element. */
void oracle_dequantize(const uint8_t *q, const float *scales, const uint8_t *zeros,
                       int64_t n, int64_t k, int group, float *w_hat) {
  const int64_t G = k / group;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n; ++r) {
    for (int64_t j = 0; j < k; ++j) {
      int64_t g = j / group;
      float d = (float)((int)q[r * k + j] - (int)zeros[r * G + g]);
      w_hat[r * k + j] = d * scales[r * G + g];
    }
  }
}

static double bf16_to_double(uint16_t h) {
  uint32_t u = ((uint32_t)h) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/*
 * Weight-only matmul y = x . W_hat^T ([SLQ-gist] Methodology 3 and Inference
 * Speedup: weights quantized, activations kept in 16-bit).  x is bf16 [m][k],
 * W_hat fp32 [n][k]; y and the error bound sum |x| |w_hat| are fp64 [m][n].
 */
void oracle_gemm(const uint16_t *x, int64_t m, int64_t k, const float *w_hat, int64_t n,
                 double *y, double *bound) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < m; ++i) {
    for (int64_t c = 0; c < n; ++c) {
      double acc = 0.0, b = 0.0;
      for (int64_t j = 0; j < k; ++j) {
        double xv = bf16_to_double(x[i * k + j]);
        double wv = (double)w_hat[c * k + j];
        acc += xv * wv;
        b += fabs(xv) * fabs(wv);
      }
      y[i * n + c] = acc;
      bound[i * n + c] = b;
    }
  }
}

/* The same products for an explicit list of (row of x, row of W_hat) pairs. */
void oracle_gemm_pairs(const uint16_t *x, int64_t k, const float *w_hat_rows,
                       const int64_t *xi, const int64_t *wi, int64_t npairs,
                       double *y, double *bound) {
#pragma omp parallel for schedule(static)
  for (int64_t p = 0; p < npairs; ++p) {
    const uint16_t *xr = x + xi[p] * k;
    const float *wr = w_hat_rows + wi[p] * k;
    double acc = 0.0, b = 0.0;
    for (int64_t j = 0; j < k; ++j) {
      double xv = bf16_to_double(xr[j]);
      double wv = (double)wr[j];
      acc += xv * wv;
      b += fabs(xv) * fabs(wv);
    }
    y[p] = acc;
    bound[p] = b;
  }
}

/*
 * Log-normalizer of a row of logits ([SLQ-blog-en] The Motivation: the
 * next-token distribution is the softmax of the logits, temperature 1):
 *   A = max_v a_v + log sum_v exp(a_v - max), in fp64.
 */
static double row_lse(const float *a, int64_t vocab) {
  double m = -INFINITY;
  for (int64_t v = 0; v < vocab; ++v)
    if ((double)a[v] > m) m = (double)a[v];
  double z = 0.0;
  for (int64_t v = 0; v < vocab; ++v) z += exp((double)a[v] - m);
  return m + log(z);
}

void oracle_row_lse(const float *a, int64_t rows, int64_t vocab, double *lse) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) lse[r] = row_lse(a + r * vocab, vocab);
}

/* Arithmetic means over rows (positions) of the per-row EAR and KL. */
static void row_means(const double *ear, const double *kl, int64_t rows, double *means) {
  double se = 0.0, sk = 0.0;
  for (int64_t r = 0; r < rows; ++r) {
    se += ear[r];
    sk += kl[r];
  }
  means[0] = rows > 0 ? se / (double)rows : 0.0;
  means[1] = rows > 0 ? sk / (double)rows : 0.0;
}

/*
 * Fidelity of a quantized model's next-token distribution q against the
 * reference p, per row (position):
 *   EAR_r = sum_v min(p_v, q_v)  ([SLQ-gist] Methodology 2, full vocabulary
 *                                 per the spec reading R9)
 *   KL_r  = sum_v p_v (log p_v - log q_v), natural log, KL(p || q)  (R10)
 * and their arithmetic means over rows (the 1/N average over positions).
 * p = softmax(a) is the reference, q = softmax(b) the quantized model.
 */
void oracle_ear_kl(const float *a, const float *b, int64_t rows, int64_t vocab,
                   double *ear, double *kl, double *means) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    const float *ar = a + r * vocab;
    const float *br = b + r * vocab;
    double A = row_lse(ar, vocab);
    double B = row_lse(br, vocab);
    double e = 0.0, d = 0.0;
    for (int64_t v = 0; v < vocab; ++v) {
      double lp = (double)ar[v] - A;
      double lq = (double)br[v] - B;
      double p = exp(lp);
      double q = exp(lq);
      e += (p < q) ? p : q;
      d += p * (lp - lq);
    }
    ear[r] = e;
    kl[r] = d;
  }
  row_means(ear, kl, rows, means);
}

/*
 * Top-K fidelity ([SLQ-gist] Methodology 2: EAR summed over the top-K tokens
 * of each position; [SLQ-readme] Evaluation: EAR and top-K KL of a model
 * against its base), at temperature T > 0:
 *   p = softmax(a / T), q = softmax(b / T) over the full vocabulary;
 *   S_r = the K tokens of largest p (equivalently largest a), ties to the
 *         lower token index (reading R16);
 *   EAR_r = sum_{v in S_r} min(p_v, q_v),
 *   KL_r  = sum_{v in S_r} p_v (log p_v - log q_v)   (natural log),
 * with no renormalization over S_r (R17), and the means over rows.
 * K = vocab and T = 1 give oracle_ear_kl.
 */
static double row_lse_t(const float *a, int64_t vocab, double T) {
  double m = -INFINITY;
  for (int64_t v = 0; v < vocab; ++v)
    if ((double)a[v] / T > m) m = (double)a[v] / T;
  double z = 0.0;
  for (int64_t v = 0; v < vocab; ++v) z += exp((double)a[v] / T - m);
  return m + log(z);
}

void oracle_ear_kl_topk(const float *a, const float *b, int64_t rows, int64_t vocab, int64_t K,
                        double T, double *ear, double *kl, double *means) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    const float *ar = a + r * vocab;
    const float *br = b + r * vocab;
    /* selection: best[0..cnt) sorted by (value desc, index asc); scanning in
       index order, a later token displaces a kept one only when strictly larger */
    int64_t best[4096];
    int64_t cnt = 0;
    for (int64_t v = 0; v < vocab; ++v) {
      if (cnt == K && !(ar[v] > ar[best[K - 1]])) continue;
      int64_t pos = (cnt < K) ? cnt : K - 1;
      while (pos > 0 && ar[v] > ar[best[pos - 1]]) {
        best[pos] = best[pos - 1];
        --pos;
      }
      best[pos] = v;
      if (cnt < K) ++cnt;
    }
    const double A = row_lse_t(ar, vocab, T);
    const double B = row_lse_t(br, vocab, T);
    double e = 0.0, d = 0.0;
    for (int64_t i = 0; i < cnt; ++i) {
      const int64_t v = best[i];
      const double lp = (double)ar[v] / T - A;
      const double lq = (double)br[v] / T - B;
      const double p = exp(lp), q = exp(lq);
      e += (p < q) ? p : q;
      d += p * (lp - lq);
    }
    ear[r] = e;
    kl[r] = d;
  }
  row_means(ear, kl, rows, means);
}

/*
 * Quantization noise of one grid over a layer, for the gamma-squared law
 * ([SLQ-gist] Methodology 1): out[0] = sum (w - w_hat)^2, out[1] = sum_g s_g^2,
 * both fp64.  Rounding noise per element scales with s^2, so the ratio of
 * out[1] between the symmetric and asymmetric grids is the predicted noise
 * ratio (R11) and the ratio of out[0] is the measured one.
 */
void oracle_quant_error(const float *W, const float *w_hat, const float *scales,
                        int64_t n, int64_t k, int group, double *out) {
  const int64_t G = k / group;
  double sse = 0.0, s2 = 0.0;
#pragma omp parallel for schedule(static) reduction(+ : sse, s2)
  for (int64_t r = 0; r < n; ++r) {
    double rs = 0.0, rq = 0.0;
    for (int64_t j = 0; j < k; ++j) {
      double e = (double)W[r * k + j] - (double)w_hat[r * k + j];
      rs += e * e;
    }
    for (int64_t g = 0; g < G; ++g) {
      double s = (double)scales[r * G + g];
      rq += s * s;
    }
    sse += rs;
    s2 += rq;
  }
  out[0] = sse;
  out[1] = s2;
}

/*
 * Storage cost in bits per parameter of a g-group format with `meta_bits` of
 * scale + zero point per group ([SLQ-readme] Search: the bit-width map adds
 * 0.156 bits per parameter at every width; Evaluation: Uniform-4 is 4.16 bpp).
 */
double oracle_bits_per_param(int bits, int meta_bits, int group) {
  return (double)bits + (double)meta_bits / (double)group;
}

/*
 * Bit-width allocation ([SLQ-summary] "3. The SLQ Pipeline": a multiple-choice
 * knapsack over the cost table, solved exactly under a budget; [SLQ-readme]
 * Pipeline: the budget is found by bisection until the target is met).
 *
 * Items l = 0..L-1 (layers or projection groups) each take exactly one of nb
 * options (bit-widths); option j of item l occupies sizes[l*nb+j] budget units
 * and costs costs[l*nb+j] (predicted degradation).  For a budget w,
 *   best(w) = min over selections with sum of sizes <= w of the sum of costs
 * (+inf when nothing fits), computed by the textbook exact recurrence over the
 * items in order:  f_0(w) = 0,  f_{l+1}(w) = min_j f_l(w - s_lj) + c_lj  over
 * the options with 0 <= s_lj <= w (a negative size marks an option that is
 * not available, R22), ties to the lower j.  best is non-increasing in
 * w, so the smallest budget in [0, W] at which something fits and best(w) <=
 * tau is found by binary search; the selection is then read back from the
 * recorded choices.
 *
 * Returns 0 when such a budget exists (budget_out = it), 1 when even W does
 * not meet tau (budget_out = -1, choice = the selection at W), 2 when nothing
 * fits in W (choice all -1).  best_out (optional) receives best(0..W).
 */
int oracle_mckp_search(int64_t L, int nb, const int64_t *sizes, const double *costs, int64_t W,
                       double tau, int32_t *choice, int64_t *budget_out, int64_t *size_out,
                       double *cost_out, double *best_out) {
  const int64_t NW = W + 1;
  double *prev = (double *)malloc(sizeof(double) * NW);
  double *cur = (double *)malloc(sizeof(double) * NW);
  int8_t *pick = (int8_t *)malloc((size_t)(L > 0 ? L : 1) * NW);
  for (int64_t w = 0; w < NW; ++w) prev[w] = 0.0;   /* no items: cost 0 at any budget */
  for (int64_t l = 0; l < L; ++l) {
    for (int64_t w = 0; w < NW; ++w) {
      double b = INFINITY;
      int j_best = -1;
      for (int j = 0; j < nb; ++j) {
        const int64_t sz = sizes[l * nb + j];
        if (sz < 0 || sz > w) continue;   /* a negative size marks an option that is never taken */
        const double v = prev[w - sz] + costs[l * nb + j];
        if (v < b) {
          b = v;
          j_best = j;
        }
      }
      cur[w] = b;
      pick[l * NW + w] = (int8_t)j_best;
    }
    double *t = prev;
    prev = cur;
    cur = t;
  }
  /* prev now holds best(0..W) */
  if (best_out)
    for (int64_t w = 0; w < NW; ++w) best_out[w] = prev[w];
  /* a budget meets the target when something fits and its best cost <= tau */
#define MEETS(w) (isfinite(prev[w]) && prev[w] <= tau)
  int status;
  int64_t budget;
  if (!MEETS(W)) {
    status = isinf(prev[W]) ? 2 : 1;
    budget = W;
  } else {
    int64_t lo = 0, hi = W;   /* invariant: budget hi meets the target */
    while (lo < hi) {
      const int64_t mid = lo + (hi - lo) / 2;
      if (MEETS(mid)) hi = mid;
      else lo = mid + 1;
    }
#undef MEETS
    status = 0;
    budget = lo;
  }
  int64_t total = 0;
  if (status == 2) {
    for (int64_t l = 0; l < L; ++l) choice[l] = -1;
  } else {
    int64_t w = budget;
    for (int64_t l = L - 1; l >= 0; --l) {
      const int j = pick[l * NW + w];
      choice[l] = j;
      w -= sizes[l * nb + j];
      total += sizes[l * nb + j];
    }
  }
  *budget_out = status == 0 ? budget : -1;
  *size_out = status == 2 ? -1 : total;
  *cost_out = status == 2 ? INFINITY : prev[budget];
  free(prev);
  free(cur);
  free(pick);
  return status;
}

/*
 * Compact group metadata ([SLQ-readme] Search: 0.156 bits per parameter of
 * metadata, i.e. 20 bits per 128-group; Evaluation: Uniform-4 at 4.16 bpp).
 * Readings R24-R27: the scale is stored in IEEE binary16, rounded UP from the
 * fp32 scale so the grid still spans [lo, hi] and the half-step bound holds;
 * the zero point and codes are computed with the stored scale; the zero point
 * takes 4 bits for b <= 4 (16 + 4 = 20 bits) and 8 bits above.
 */

/* Value of binary16 bits (positive, finite), from the format's definition:
 * exponent field e, fraction f: e == 0 -> f * 2^-24, else (1 + f/1024) 2^(e-15). */
double oracle_f16_value(uint16_t bits) {
  const int e = (bits >> 10) & 31, f = bits & 1023;
  if (e == 0) return ldexp((double)f, -24);
  return ldexp(1.0 + (double)f / 1024.0, e - 15);
}

/* The smallest binary16 value >= s (s > 0, finite), as bits; values above
 * 65504 saturate at 65504.  The spacing of binary16 around s is 2^(E - 10)
 * for 2^E <= s < 2^(E+1), E >= -14, and 2^-24 below 2^-14; s / spacing is
 * exact in fp64, so ceil() gives the round-up exactly. */
uint16_t oracle_f16_round_up(float s) {
  const double v = (double)s;
  if (v >= 65504.0) return 0x7BFF;
  int e2;
  frexp(v, &e2);   /* v = f * 2^e2, f in [0.5, 1): 2^(e2-1) <= v < 2^e2 */
  const int E = e2 - 1;
  const double spacing = E < -14 ? ldexp(1.0, -24) : ldexp(1.0, E - 10);
  const double r = ceil(v / spacing) * spacing;
  if (r < ldexp(1.0, -14)) return (uint16_t)(r / ldexp(1.0, -24));   /* subnormal */
  int er;
  frexp(r, &er);
  const int Er = er - 1;
  const int frac = (int)((r / ldexp(1.0, Er) - 1.0) * 1024.0);
  return (uint16_t)(((Er + 15) << 10) | frac);
}

/* Zero-point bits of the compact layout: 4 for b <= 4, else 8. */
int oracle_compact_zero_bits(int bits) { return bits <= 4 ? 4 : 8; }

/*
 * Asymmetric (or symmetric) group quantization with compact metadata: the
 * steps of oracle_quantize, except that s is replaced by the binary16 value
 * rounded up from it before z and q are computed.  scales16[i] holds its
 * bits and zeros[i] the zero point (one byte per group, unpacked; see
 * oracle_pack_zeros), i = row * G + g.
 */
void oracle_quantize_compact(const float *W, int64_t n, int64_t k, int bits, int group,
                             int symmetric, uint8_t *q, uint16_t *scales16, uint8_t *zeros) {
  const int maxq = (1 << bits) - 1;
  const int64_t G = k / group;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n; ++r) {
    for (int64_t g = 0; g < G; ++g) {
      const float *w = W + r * k + g * group;
      float s, lo = 0.0f;
      int z;
      if (!symmetric) {
        float hi = 0.0f;
        for (int i = 0; i < group; ++i) {
          if (w[i] < lo) lo = w[i];
          if (w[i] > hi) hi = w[i];
        }
        s = (hi - lo) / (float)maxq;
      } else {
        float m = 0.0f;
        for (int i = 0; i < group; ++i) {
          float a = fabsf(w[i]);
          if (a > m) m = a;
        }
        s = (2.0f * m) / (float)maxq;
      }
      uint16_t h;
      if (s == 0.0f) {
        h = 0x3C00; /* 1.0 */
        s = 1.0f;
        z = symmetric ? 1 << (bits - 1) : 0;
      } else {
        h = oracle_f16_round_up(s);
        s = (float)oracle_f16_value(h);
        z = symmetric ? 1 << (bits - 1) : (int)clamp_code(rintf(-lo / s), maxq);
      }
      scales16[r * G + g] = h;
      zeros[r * G + g] = (uint8_t)z;
      for (int i = 0; i < group; ++i) {
        const float tq = rintf(w[i] / s);
        q[r * k + g * group + i] = (uint8_t)(int)clamp_code(tq + (float)z, maxq);
      }
    }
  }
}

/* Zero points of `count` groups in the compact layout: nibble i of the byte
 * stream (low nibble first) for b <= 4, else byte i.  Returns bytes written. */
int64_t oracle_pack_zeros(const uint8_t *zeros, int64_t count, int bits, uint8_t *out) {
  if (oracle_compact_zero_bits(bits) == 8) {
    for (int64_t i = 0; i < count; ++i) out[i] = zeros[i];
    return count;
  }
  const int64_t nb = (count + 1) / 2;
  for (int64_t i = 0; i < nb; ++i) out[i] = 0;
  for (int64_t i = 0; i < count; ++i) out[i / 2] |= (uint8_t)((zeros[i] & 15) << (4 * (i % 2)));
  return nb;
}

/* Reconstruction from compact metadata: w_hat = fl32((q - z) * s), s the
 * binary16 scale's value, z read from the packed zero points. */
void oracle_dequantize_compact(const uint8_t *q, const uint16_t *scales16, const uint8_t *zpacked,
                               int64_t n, int64_t k, int group, int bits, float *w_hat) {
  const int64_t G = k / group;
  const int zb = oracle_compact_zero_bits(bits);
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n; ++r) {
    for (int64_t j = 0; j < k; ++j) {
      const int64_t i = r * G + j / group;
      const int z = zb == 8 ? zpacked[i] : (zpacked[i / 2] >> (4 * (i % 2))) & 15;
      const float s = (float)oracle_f16_value(scales16[i]);
      float d = (float)((int)q[r * k + j] - z);
      w_hat[r * k + j] = d * s;
    }
  }
}

/*
 * GPTQ column pass in fp32 with lazy block updates.  The pages name GPTQ as
 * the code-choice step ([SLQ-readme] Pipeline paragraph: layer-wise GPTQ at
 * every bit-width, asymmetric INT, group 128) without defining it; the steps
 * are those of the published algorithm (Frantar, Ashkboos, Hoefler, Alistarh,
 * "GPTQ", ICLR 2023, Algorithm 1: quantize the columns in order, divide each
 * column's error by the diagonal of the inverse-Hessian factor, move the
 * block's later columns at once and every later column once per block).
 *
 * In : W fp32 [n][k]; U fp32 [k][k] upper triangular with U^T U = H^-1
 *      (entries below the diagonal are never read); dead [k] or NULL
 *      (nonzero: an input that never fires, whose weight column is zero).
 * Out: q [n][k] codes, scales fp32 [n][G], zeros [n][G].
 * Readings (R28-R32 in the design notes):
 *   - the lazy block is the 128-group, so each group's scale and zero point
 *     come from its current (already moved) weights at its first column, by
 *     the plain quantizer's fp32 steps (R1-R4 above);
 *   - every operation is one fp32 rounding, in this order: for column i of
 *     the block, e_i = fl32(fl32(w_i - w_hat_i) / U_ii), then each later
 *     column j of the block takes w_j = fma(-e_i, U_ij, w_j); after the block
 *     every later column c takes w_c = fl32(w_c - a_c) with a_c the fma chain
 *     a = fma(e_p, U[i1 + p][c], a) over p = 0, 1, ..., 127 from a = 0.
 * Rows are independent given U.
 */
void oracle_gptq_columns(const float *W, const float *U, const uint8_t *dead, int64_t n,
                         int64_t k, int bits, int group, uint8_t *q, float *scales,
                         uint8_t *zeros) {
  const int maxq = (1 << bits) - 1;
  const int64_t G = k / group;
#pragma omp parallel
  {
    float *w = (float *)malloc((size_t)k * sizeof(float));
    float *e = (float *)malloc((size_t)group * sizeof(float));
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < n; ++r) {
      for (int64_t c = 0; c < k; ++c) w[c] = (dead && dead[c]) ? 0.0f : W[r * k + c];
      for (int64_t g = 0; g < G; ++g) {
        const int64_t i1 = g * group;
        /* group parameters from the current weights (R1-R4) */
        float glo = 0.0f, ghi = 0.0f;
        for (int p = 0; p < group; ++p) {
          if (w[i1 + p] < glo) glo = w[i1 + p];
          if (w[i1 + p] > ghi) ghi = w[i1 + p];
        }
        const float grange = ghi - glo;
        float s = grange / (float)maxq;
        int z;
        if (s == 0.0f) {
          s = 1.0f;
          z = 0;
        } else {
          z = (int)clamp_code(rintf((-glo) / s), maxq);
        }
        scales[r * G + g] = s;
        zeros[r * G + g] = (uint8_t)z;
        /* the block's columns in order, moving the block's later columns */
        for (int p = 0; p < group; ++p) {
          const int64_t i = i1 + p;
          const float rq = rintf(w[i] / s);
          int qi = (int)clamp_code(rq + (float)z, maxq);
          q[r * k + i] = (uint8_t)qi;
          float w_hat = (float)(qi - z) * s;
          float d = w[i] - w_hat;
          e[p] = d / U[i * k + i];
          for (int64_t j = i + 1; j < i1 + group; ++j) w[j] = fmaf(-e[p], U[i * k + j], w[j]);
        }
        /* every later column once, by the block's errors */
        for (int64_t c = i1 + group; c < k; ++c) {
          float a = 0.0f;
          for (int p = 0; p < group; ++p) a = fmaf(e[p], U[(i1 + p) * k + c], a);
          w[c] = w[c] - a;
        }
      }
    }
    free(w);
    free(e);
  }
}
