/*
 * slq.h -- C ABI of libslq.so, the MI355X (gfx950) hot path of SLQ
 * (Statistically-Lossless Quantization): asymmetric INT2..INT8 group-128
 * weight quantization with dense bit-packing, the weight-only dequantize
 * matmul (W{2..8}A16) that serves a layer-wise mixed-bit-width model, and
 * the EAR / KL fidelity reductions used to judge it.
 *
 * Sources (page title -> section):
 *   gist.science, "Statistically-Lossless Quantization of Large Language
 *     Models": Methodology 1 (centering inefficiency gamma = 2M/R and the
 *     gamma-squared variance law), Methodology 2 (EAR), Methodology 3
 *     (asymmetric integer group quantization, group size 128; served by
 *     weight-only mixed-precision kernels), Inference Speedup.
 *   "SLQ" GitHub README: Pipeline (asymmetric INT, g128, bit-widths 2..8),
 *     Usage 4 (weights packed to their per-layer bit-width on load),
 *     Evaluation (EAR and KL of a model against its base).
 *
 * Conventions shared by every entry point
 *   - Every data pointer is a DEVICE pointer (hipMalloc / torch CUDA memory)
 *     owned by the caller; the library never allocates, frees or retains it.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues work on that stream and returns; results are visible after the
 *     stream is synchronized.  Device faults surface at that synchronization.
 *   - Arguments are validated on the host before any HIP call.  On any
 *     status other than SLQ_OK nothing was enqueued and outputs are untouched.
 *   - Sizes may be zero (then the call is a no-op returning SLQ_OK).
 *   - Calls on different streams are independent and thread-safe; calls that
 *     share a workspace buffer must be ordered by the caller.
 *   - Non-finite weights or logits are a precondition violation (results are
 *     unspecified, never an error code).
 */
#ifndef SLQ_H
#define SLQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SLQ_OK = 0,
  SLQ_EINVAL = 1,   /* bad size, bit-width, pointer, alignment or aliasing   */
  SLQ_ENOTSUP = 2,  /* valid request the library does not implement (g!=128) */
  SLQ_EHIP = 3,     /* the HIP runtime reported an error at launch            */
  SLQ_ESCRATCH = 4  /* slq_dequant_gemm_noalloc: the request needs more split-k
                       scratch than the static array holds                   */
} slq_status;

typedef enum {
  SLQ_ASYM = 0,     /* asymmetric grid: scale and zero point per group       */
  SLQ_SYM = 1       /* symmetric grid (comparison only): center 2^(b-1)      */
} slq_grid;

typedef enum {
  SLQ_META_F32 = 0,     /* fp32 scale + uint8 zero point per group (40 bits)      */
  SLQ_META_COMPACT = 1  /* binary16 scale rounded up + 4-bit zero point (b <= 4,
                           20 bits per group) or 8-bit zero point (b >= 5)       */
} slq_meta;

typedef void *slq_stream; /* a hipStream_t */

/*
 * A quantized weight W[n][k] (n outputs, k inputs, k contiguous) in groups of
 * `group` consecutive inputs along k.  G = k / group groups per row.
 *   codes  : uint32 [n][k*bits/32].  Each row is one little-endian bitstream:
 *            code j of the row occupies bits [j*bits, j*bits+bits) of the
 *            integer sum_i codes[row][i] * 2^(32 i); group g starts at word
 *            4*bits*g.  For bits = 4 this is 8 codes per word, nibble j = code
 *            j; 3/5/6/7-bit codes straddle word boundaries with no padding.
 *   scales, zeros: group metadata, flat group index i = row * G + g, in one of
 *   two layouts (`meta`):
 *   SLQ_META_F32     scales fp32 [n*G] (> 0), zeros uint8 [n*G] in
 *                    [0, 2^bits - 1]: bits + 40/group bits per parameter.
 *   SLQ_META_COMPACT scales binary16 [n*G]: the fp32 scale rounded up to the
 *                    next binary16 value (so the half-step error bound still
 *                    holds), and the zero point and codes are computed with that
 *                    scale; zeros: 4-bit nibbles for bits <= 4 (nibble i of the
 *                    byte stream, low nibble first: ceil(n*G/2) bytes), bytes
 *                    for bits >= 5.  bits + 20/group bits per parameter for
 *                    bits <= 4, the README's 0.156 bpp of metadata (Search:
 *                    bit-width map; Evaluation: Uniform-4 at 4.16 bpp), and
 *                    bits + 24/group above.  Scales beyond the binary16 range
 *                    (65504) saturate; no weight of a real model comes near.
 * Reconstruction: w_hat[n][k] = fl32((q[n][k] - z[i]) * s[i]), s in fp32.
 * Alignment: codes and scales 16 bytes, zeros 4 bytes.
 */
typedef struct {
  int32_t bits;   /* 2..8                                   */
  int32_t group;  /* 128                                    */
  int64_t n;      /* rows (outputs)                         */
  int64_t k;      /* columns (inputs), a multiple of group  */
  uint32_t *codes;
  void *scales;   /* fp32 or binary16, per `meta`           */
  uint8_t *zeros;
  int32_t meta;   /* slq_meta                               */
  int32_t reserved;
} slq_packed;

/* Bytes of the codes array: n*k*bits/8 (0 on invalid arguments). */
size_t slq_codes_bytes(int64_t n, int64_t k, int bits);
/* Bytes of the scales and zeros arrays for a metadata layout (0 on invalid
 * arguments; group 128). */
size_t slq_scales_bytes(int64_t n, int64_t k, int32_t meta);
size_t slq_zeros_bytes(int64_t n, int64_t k, int bits, int32_t meta);

/*
 * Group quantization and dense packing of an fp32 weight (gist.science
 * summary, Methodology 3: asymmetric integer group quantization with group
 * size 128; README, Pipeline: bit-widths 2..8; README, Usage 4: packing to
 * the per-layer bit-width).  Per row n and group g, with maxq = 2^bits - 1:
 *   SLQ_ASYM: lo = min(0, min w), hi = max(0, max w);
 *             s = fl32(fl32(hi - lo) / maxq); if s == 0 then s = 1, z = 0;
 *             else z = clamp(rint(fl32(-lo / s)), 0, maxq).
 *   SLQ_SYM : M = max |w|, s = fl32(2M / maxq) (1 if zero), z = 2^(bits-1)
 *             (the comparison grid of Methodology 1).
 *   q = clamp(rint(fl32(w / s)) + z, 0, maxq); rint rounds half to even and
 *   every fp32 operation is IEEE correctly rounded, so the result is exact
 *   and reproducible bit for bit.  With out->meta = SLQ_META_COMPACT, s is
 *   rounded up to binary16 before z and q are computed.
 * In : W fp32 [n][k] (device, 16-byte aligned), n >= 0, k % group == 0,
 *      bits in 2..8, group == 128 (else SLQ_ENOTSUP).
 * Out: out->meta selects the metadata layout; out->codes/scales/zeros must
 *      point to caller-owned device buffers of slq_codes_bytes(n,k,bits),
 *      slq_scales_bytes(n,k,meta) and slq_zeros_bytes(n,k,bits,meta) bytes,
 *      aligned as above, none overlapping W.  The call fills out->bits,
 *      group, n and k and writes the three arrays.
 */
slq_status slq_quantize_pack(const float *W, int64_t n, int64_t k, int bits, int group,
                             slq_grid grid, slq_packed *out, slq_stream stream);

/*
 * Reconstruction w_hat[n][k] = fl32((q - z) * s) into W_deq (fp32 [n][k],
 * device, not overlapping the packed arrays).
 */
slq_status slq_dequantize(const slq_packed *w, float *W_deq, slq_stream stream);

/* Workspace bytes slq_dequant_gemm needs for this (m, w); may be 0. */
size_t slq_gemm_workspace_bytes(int64_t m, const slq_packed *w);

/*
 * Weight-only dequantize matmul y[m][n] = sum_k x[m][k] * w_hat[n][k]
 * (gist.science summary, Methodology 3 and Inference Speedup: 16-bit
 * activations against the packed low-bit weights of each layer).
 * In : x bf16 bit patterns [m][k] (device, 16-byte aligned), w a packed
 *      weight from slq_quantize_pack (any bits 2..8), m >= 0.
 * Out: y fp32 [m][n] (device, 16-byte aligned, not overlapping inputs).
 * workspace: device buffer of slq_gemm_workspace_bytes(m, w) bytes, 256-byte
 *      aligned, ZERO-FILLED before its first use.  Its first 64 KiB hold
 *      split-K tickets that every completed call leaves at zero, so one buffer
 *      (of the largest size needed) serves any sequence of calls on one
 *      stream; calls that overlap in time must not share it.  Split-K partial
 *      sums (decode, and prefill grids too small to fill the chip) follow the
 *      tickets and are overwritten by every call.  May be NULL when the size
 *      is 0.
 * Accumulation is fp32.  m <= 64 runs the decode kernel (exact integer
 * (q - z), per-group scale in fp32); m > 64 runs the prefill kernel (w_hat
 * rounded to bf16 in registers, activations staged in LDS, bf16 MFMA).
 * Both stay within |y - y_exact| <= 1e-2 * sum_k |x||w_hat|; split-K sums
 * are taken in a fixed order, so repeated calls are bit-identical.
 */
slq_status slq_dequant_gemm(const uint16_t *x_bf16, const slq_packed *w, int64_t m,
                            float *y, void *workspace, slq_stream stream);

/* Bytes of the static split-k scratch array slq_dequant_gemm_noalloc uses per GPU. */
size_t slq_noalloc_scratch_bytes(void);

/*
 * slq_dequant_gemm for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * kernels and results, with the split-k scratch taken from a static device
 * array of slq_noalloc_scratch_bytes() bytes (32 MiB) instead of a caller
 * workspace.  The library holds one such array on every GPU it runs on until
 * the process ends; the first call on a device looks up its address and
 * clears its ticket area with a fill kernel on `stream`.  The call allocates
 * nothing (no hipMalloc, no library allocation).  Calls on one GPU share its
 * array: calls that overlap in time on the same GPU (other streams, other
 * threads) race and must be ordered by the caller.
 * Errors: as slq_dequant_gemm, and SLQ_ESCRATCH (nothing enqueued) when
 * slq_gemm_workspace_bytes(m, w) exceeds the array.
 */
slq_status slq_dequant_gemm_noalloc(const uint16_t *x_bf16, const slq_packed *w, int64_t m,
                                    float *y, slq_stream stream);

/*
 * Name of the kernel instance slq_dequant_gemm launches for (m, w), as the
 * profiler reports it (e.g. "slq::gemv_kernel<4, 1, 1, 4>"), so tools can
 * match per-kernel statistics to calls.  Static storage; "" on invalid
 * arguments.
 */
const char *slq_dequant_gemm_kernel_name(int64_t m, const slq_packed *w);

/* Workspace bytes slq_ear_kl / slq_row_lse need for (rows, vocab). */
size_t slq_ear_kl_workspace_bytes(int64_t rows, int64_t vocab);

/*
 * Row log-normalizer lse[r] = max_v a[r][v] + log sum_v exp(a[r][v] - max),
 * fp64 out (the softmax at temperature 1 that defines the next-token
 * distribution; SLQ blog, The Motivation).
 * In : a fp32 [rows][vocab] (device, 16-byte aligned).  Out: lse fp64 [rows].
 * workspace: slq_ear_kl_workspace_bytes(rows, vocab) bytes, 256-byte aligned.
 */
slq_status slq_row_lse(const float *logits, int64_t rows, int64_t vocab, double *lse,
                       void *workspace, slq_stream stream);

/*
 * Fidelity of a quantized model's next-token distributions q = softmax(b)
 * against the reference p = softmax(a), per row (position):
 *   EAR_r = sum_v min(p_v, q_v)    (gist.science summary, Methodology 2; over
 *                                   the full vocabulary)
 *   KL_r  = sum_v p_v log(p_v / q_v), natural log (README, Evaluation)
 * and means[0] = mean_r EAR_r, means[1] = mean_r KL_r.
 * In : logits_p (reference), logits_q: fp32 [rows][vocab] (device, 16-byte
 *      aligned).  Out: ear_rows, kl_rows fp32 [rows]; means fp64 [2].
 * workspace: slq_ear_kl_workspace_bytes(rows, vocab) bytes, 256-byte aligned.
 * Reductions are deterministic (fixed order): repeated calls are bit-equal.
 */
slq_status slq_ear_kl(const float *logits_p, const float *logits_q, int64_t rows, int64_t vocab,
                      float *ear_rows, float *kl_rows, double *means, void *workspace,
                      slq_stream stream);

/* Largest K slq_ear_kl_topk accepts. */
#define SLQ_TOPK_MAX 64

/*
 * Top-K fidelity at a temperature (gist.science summary, Methodology 2: EAR
 * taken over the top-K tokens of each position; README, Evaluation: top-K KL).
 * With p = softmax(a / T), q = softmax(b / T) over the full vocabulary and
 * S_r the K tokens with the largest reference logits a[r][.] (equal logits:
 * the lower token index first):
 *   EAR_r = sum_{v in S_r} min(p_v, q_v)
 *   KL_r  = sum_{v in S_r} p_v log(p_v / q_v)      (no renormalization over S_r)
 * and means[0] = mean_r EAR_r, means[1] = mean_r KL_r.  K = vocab gives the
 * full-vocabulary metrics of slq_ear_kl.
 * In : logits_p (reference), logits_q: fp32 [rows][vocab] (device, 16-byte
 *      aligned); 1 <= K <= min(vocab, SLQ_TOPK_MAX); temperature finite, > 0.
 * Out: ear_rows, kl_rows fp32 [rows]; means fp64 [2].
 * workspace: slq_ear_kl_workspace_bytes(rows, vocab) bytes, 256-byte aligned.
 * Errors: SLQ_EINVAL for K or temperature out of range and for the argument
 * faults slq_ear_kl rejects.  Deterministic: repeated calls are bit-equal.
 */
slq_status slq_ear_kl_topk(const float *logits_p, const float *logits_q, int64_t rows,
                           int64_t vocab, int64_t K, double temperature, float *ear_rows,
                           float *kl_rows, double *means, void *workspace, slq_stream stream);

/* Workspace bytes slq_gptq_quantize needs for W[n][k]. */
size_t slq_gptq_workspace_bytes(int64_t n, int64_t k);

/*
 * GPTQ code selection (named by the README, Pipeline, as the code-choice step:
 * layer-wise GPTQ at every bit-width, asymmetric INT, group size 128; steps of
 * the published algorithm, Frantar et al., ICLR 2023, Algorithm 1 with the
 * Cholesky form of the inverse Hessian):
 *   dead inputs (H_ii = 0) get H_ii = 1 and a zeroed weight column;
 *   H += damp * mean(diag H) * I;  U upper with U^T U = H^-1 (fp64);
 *   for each column i: at a group's first column its scale and zero point come
 *   from the group's current weights (the slq_quantize_pack steps), the column
 *   is quantized, and the later columns move by -err_i * U[i][j] with
 *   err_i = (w_i - w_hat_i) / U[i][i]  (weights updated in fp32).
 * It is slq_gptq_factor followed by slq_gptq_columns on the fp32 U (their
 * comments give the exact operation order).
 * In : W fp32 [n][k], H fp32 [k][k] symmetric positive semi-definite (the
 *      layer Hessian 2 X X^T; device, 16-byte aligned), 1 <= n, 128 <= k <=
 *      32768, k % 128 == 0, bits 2..8, group 128, damp > 0 and finite.
 * Out: out as for slq_quantize_pack with out->meta = SLQ_META_F32 (the
 *      compact layout: SLQ_ENOTSUP); u_out fp64 [k][k] or NULL: U.
 * workspace: slq_gptq_workspace_bytes(n, k) bytes, 256-byte aligned.
 * If H + damping is not positive definite the factor holds NaN and so do the
 * scales; nothing else is reported.
 */
slq_status slq_gptq_quantize(const float *W, const float *H, int64_t n, int64_t k, int bits,
                             int group, double damp, slq_packed *out, double *u_out,
                             void *workspace, slq_stream stream);

/* Workspace bytes slq_gptq_factor needs for a k x k Hessian (0 if k is invalid). */
size_t slq_gptq_factor_workspace_bytes(int64_t k);

/*
 * The inverse-Hessian factor of GPTQ alone (steps 1-2 of slq_gptq_quantize),
 * so that one factor serves a layer at every bit-width (README, Pipeline:
 * layer-wise GPTQ at each bit-width 2..8 against the same calibration data):
 *   dead[i] = (H_ii == 0); dead inputs get H_ii = 1;
 *   H += damp * mean(diag H) * I;  U upper triangular with U^T U = H^-1,
 *   computed in fp64 and written rounded to fp32 (zeros below the diagonal).
 * In : H fp32 [k][k] symmetric positive semi-definite (device, 16-byte
 *      aligned), 128 <= k <= 32768, k % 128 == 0, damp > 0 and finite.
 * Out: U fp32 [k][k] (16-byte aligned), dead uint8 [k], u_out fp64 [k][k]
 *      (8-byte aligned) or NULL: U before rounding.  No output may overlap H
 *      or another output.
 * workspace: slq_gptq_factor_workspace_bytes(k) bytes, 256-byte aligned.
 * If H + damping is not positive definite U holds NaN.
 */
slq_status slq_gptq_factor(const float *H, int64_t k, double damp, float *U, uint8_t *dead,
                           double *u_out, void *workspace, slq_stream stream);

/* Workspace bytes slq_gptq_columns needs for W[n][k] (0 if invalid). */
size_t slq_gptq_columns_workspace_bytes(int64_t n, int64_t k);

/*
 * The GPTQ column pass alone (step 3 of slq_gptq_quantize), given the fp32
 * factor U of slq_gptq_factor (or any upper-triangular U with a nonzero
 * diagonal; entries below the diagonal are never read).  Lazy blocks of the
 * 128-group, fp32 with one rounding per operation, in this order: the
 * working weights are W with the columns of dead inputs set to 0; per group
 * (first column i1) the scale and zero point come from the group's current
 * weights by the slq_quantize_pack steps; for each column i of the group,
 * ascending: q_i = clamp(rint(w_i / s) + z), e_i = fl32(fl32(w_i - w_hat_i) /
 * U_ii), and every later column j of the group takes w_j = fma(-e_i, U_ij,
 * w_j); then every column c after the group takes w_c = fl32(w_c - a_c),
 * a_c = fma(e_p, U[i1 + p][c], a) chained over p = 0..127 from a = 0.
 * Results are bit-identical across calls.
 * In : W fp32 [n][k], U fp32 [k][k] (device, 16-byte aligned), dead uint8
 *      [k] or NULL (nonzero = dead input), n >= 1, k as for slq_gptq_factor,
 *      bits 2..8, group 128 (else SLQ_ENOTSUP).
 * Out: out as for slq_gptq_quantize (out->meta must be SLQ_META_F32), not
 *      overlapping the inputs.
 * workspace: slq_gptq_columns_workspace_bytes(n, k) bytes, 256-byte aligned.
 */
slq_status slq_gptq_columns(const float *W, const float *U, const uint8_t *dead, int64_t n,
                            int64_t k, int bits, int group, slq_packed *out, void *workspace,
                            slq_stream stream);

/* Workspace bytes slq_mckp_search needs for L items and budgets 0..W. */
size_t slq_mckp_workspace_bytes(int64_t L, int64_t W);

/*
 * Bit-width allocation (gist.science summary, 3. The SLQ Pipeline: a
 * multiple-choice knapsack over the cost table solved exactly under a bit
 * budget; README, Pipeline: the budget is searched by bisection until the
 * target is met).
 * Item l (a layer or projection) takes exactly one of nb options (bit-widths);
 * option j occupies sizes[l*nb+j] budget units and costs costs[l*nb+j]
 * (predicted degradation).  best(w) = least total cost with total size <= w
 * (+inf when nothing fits), exact for every w in 0..W; the result is the
 * smallest budget with best(w) finite and <= tau, and the selection attaining
 * it (equal costs: the lower option index, read back from the last item).
 * In : sizes int64 [L][nb] (device; negative sizes are never selected),
 *      costs fp64 [L][nb] (device), 1 <= L, 1 <= nb <= 127, 0 <= W < 2^31 - 1,
 *      tau not NaN.
 * Out: choice int32 [L] (option per item, -1 when nothing fits in W);
 *      result int64 [3] = {status, budget, size}: status 0 found, 1 even W
 *      misses tau (budget -1, choice = the selection at W), 2 nothing fits
 *      (budget and size -1); cost fp64 [1] = best(budget), or best(W);
 *      best fp64 [W+1] or NULL: best(0..W).
 * workspace: slq_mckp_workspace_bytes(L, W) bytes, 256-byte aligned.
 * Deterministic and bit-identical across calls (fp64 sums in item order).
 */
slq_status slq_mckp_search(const int64_t *sizes, const double *costs, int64_t L, int32_t nb,
                           int64_t W, double tau, int32_t *choice, int64_t *result, double *cost,
                           double *best, void *workspace, slq_stream stream);

/* Workspace bytes slq_quant_error needs for w. */
size_t slq_quant_error_workspace_bytes(const slq_packed *w);

/*
 * Quantization noise of a grid over a layer, for the gamma-squared law
 * (gist.science summary, Methodology 1): out[0] = sum (w - w_hat)^2,
 * out[1] = sum_g s_g^2, fp64, deterministic order.  The symmetric/asymmetric
 * ratio of out[0] is the measured noise-variance ratio, that of out[1] the
 * predicted one (rounding noise is s^2/12 per element).
 * In : W fp32 [n][k] (the quantized source), w packed from W.
 * Out: out fp64 [2] (device).
 */
slq_status slq_quant_error(const float *W, const slq_packed *w, double *out, void *workspace,
                           slq_stream stream);

/* Words of `folds` slq_stream_read writes for `bytes` bytes (one per 16 KiB). */
size_t slq_stream_read_words(size_t bytes);

/*
 * Measurement aid (not part of the method): one plain read of `bytes` bytes
 * of the device buffer `buf` with coalesced 16-byte loads, 1024 consecutive
 * 16-byte words per workgroup; workgroup i writes the XOR of the 32-bit words
 * it read to folds[i] (bytes past the end read as zero).  Timing it over
 * buffers of the decode layers' sizes gives the read ceiling and per-launch
 * floor that a dequant-GEMV of the same bytes could at best reach.
 * bytes % 16 == 0; buf 16-byte aligned; folds: device uint32
 * [slq_stream_read_words(bytes)], 4-byte aligned, outside buf.
 */
slq_status slq_stream_read(const void *buf, size_t bytes, uint32_t *folds, slq_stream stream);

/* Static description of a status code. */
const char *slq_strerror(slq_status s);

#ifdef __cplusplus
}
#endif
#endif /* SLQ_H */
