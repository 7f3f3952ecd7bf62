// C ABI of libslq: argument validation on the host, then the HIP launchers.
// Every check runs before the first HIP call, so an invalid request returns
// SLQ_EINVAL / SLQ_ENOTSUP with nothing enqueued and outputs untouched.
#include <cmath>
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdio.h>

#include "../../include/slq.h"
#include "launch.h"

namespace {

constexpr int kGroupSize = 128;                 // group size the kernels are built for
constexpr int64_t kMaxDim = (int64_t)1 << 31;   // kernels index rows/cols with int
#ifndef SLQ_DECODE_MAX_M
#define SLQ_DECODE_MAX_M 64
#endif
constexpr int64_t kDecodeMaxM = SLQ_DECODE_MAX_M;   // activation rows served by the decode kernels

bool aligned(const void *p, size_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

bool overlap(const void *a, size_t na, const void *b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const char *pa = static_cast<const char *>(a), *pb = static_cast<const char *>(b);
  return pa < pb + nb && pb < pa + na;
}

slq_status from_hip(hipError_t e) { return e == hipSuccess ? SLQ_OK : SLQ_EHIP; }

bool dims_ok(int64_t n, int64_t k) {
  return n >= 0 && k >= 0 && n < kMaxDim && k < kMaxDim && (n == 0 || k <= ((int64_t)1 << 50) / n);
}

struct PackedSizes {
  size_t codes, scales, zeros;
};

PackedSizes sizes_of(int64_t n, int64_t k, int bits, int group, int32_t meta) {
  PackedSizes s;
  const size_t groups = (size_t)(n * (k / group));
  s.codes = (size_t)(n * k / 8 * bits);
  s.scales = groups * (meta == SLQ_META_COMPACT ? 2 : 4);
  s.zeros = meta == SLQ_META_COMPACT && bits <= 4 ? (groups + 1) / 2 : groups;
  return s;
}

bool meta_ok(int32_t meta) { return meta == SLQ_META_F32 || meta == SLQ_META_COMPACT; }

// Shape, bit-width, group, pointers and alignment of a packed weight.
slq_status check_packed(const slq_packed *w, PackedSizes *sz) {
  if (!w) return SLQ_EINVAL;
  if (w->bits < 2 || w->bits > 8) return SLQ_EINVAL;
  if (w->group <= 0) return SLQ_EINVAL;
  if (w->group != kGroupSize) return SLQ_ENOTSUP;
  if (!dims_ok(w->n, w->k) || w->k % w->group != 0 || !meta_ok(w->meta)) return SLQ_EINVAL;
  *sz = sizes_of(w->n, w->k, w->bits, w->group, w->meta);
  if (w->n * w->k > 0) {
    if (!w->codes || !w->scales || !w->zeros) return SLQ_EINVAL;
    if (!aligned(w->codes, 16) || !aligned(w->scales, 16) || !aligned(w->zeros, 4))
      return SLQ_EINVAL;
    if (overlap(w->codes, sz->codes, w->scales, sz->scales) ||
        overlap(w->codes, sz->codes, w->zeros, sz->zeros) ||
        overlap(w->scales, sz->scales, w->zeros, sz->zeros))
      return SLQ_EINVAL;
  }
  return SLQ_OK;
}

}  // namespace

namespace {

constexpr size_t kScratchBytes = slq::kNoallocScratchBytes;

size_t gemm_ws_bytes(int64_t m, const slq_packed *w);

// Validation and launch shared by slq_dequant_gemm and its allocation-free
// variant (noalloc: the workspace is the device's scratch array).
slq_status dequant_gemm_checked(const uint16_t *x_bf16, const slq_packed *w, int64_t m, float *y,
                                void *workspace, bool noalloc, slq_stream stream) {
  PackedSizes sz;
  slq_status st = check_packed(w, &sz);
  if (st != SLQ_OK) return st;
  if (m < 0 || m >= kMaxDim) return SLQ_EINVAL;
  if (m == 0 || w->n == 0) return SLQ_OK;
  const size_t xb = (size_t)(m * w->k) * 2, yb = (size_t)(m * w->n) * sizeof(float);
  if (!y || !aligned(y, 16)) return SLQ_EINVAL;
  if (xb > 0 && (!x_bf16 || !aligned(x_bf16, 16))) return SLQ_EINVAL;
  const size_t wsb = gemm_ws_bytes(m, w);
  if (noalloc) {
    if (wsb > kScratchBytes) return SLQ_ESCRATCH;
  } else if (wsb > 0 && (!workspace || !aligned(workspace, 256))) {
    return SLQ_EINVAL;
  }
  if (overlap(y, yb, x_bf16, xb) || overlap(y, yb, w->codes, sz.codes) ||
      overlap(y, yb, w->scales, sz.scales) || overlap(y, yb, w->zeros, sz.zeros) ||
      overlap(y, yb, workspace, wsb) || overlap(workspace, wsb, x_bf16, xb) ||
      overlap(workspace, wsb, w->codes, sz.codes) ||
      overlap(workspace, wsb, w->scales, sz.scales) || overlap(workspace, wsb, w->zeros, sz.zeros))
    return SLQ_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  slq::GemvPlan plan{};
  if (m <= kDecodeMaxM) {
    plan = slq::gemv_plan(m, w->n, w->k, w->bits);
    if (plan.ksplits == 0) return SLQ_ENOTSUP;
  }
  if (noalloc && wsb > 0) {
    const hipError_t e = slq::noalloc_scratch(&workspace, s);
    if (e != hipSuccess) return SLQ_EHIP;
  }
  if (m <= kDecodeMaxM)
    return from_hip(slq::launch_gemv(x_bf16, w->codes, w->scales, w->zeros,
                                     w->meta == SLQ_META_COMPACT, m, w->n, w->k, w->bits, y,
                                     workspace, plan, s));
  return from_hip(slq::launch_gemm(x_bf16, w->codes, w->scales, w->zeros,
                                   w->meta == SLQ_META_COMPACT, m, w->n, w->k, w->bits, y,
                                   workspace, s));
}

}  // namespace

extern "C" {

size_t slq_codes_bytes(int64_t n, int64_t k, int bits) {
  if (bits < 2 || bits > 8 || !dims_ok(n, k) || k % 32 != 0) return 0;
  return (size_t)(n * k / 8 * bits);
}

size_t slq_scales_bytes(int64_t n, int64_t k, int32_t meta) {
  if (!dims_ok(n, k) || k % kGroupSize != 0 || !meta_ok(meta)) return 0;
  return sizes_of(n, k, 8, kGroupSize, meta).scales;
}

size_t slq_zeros_bytes(int64_t n, int64_t k, int bits, int32_t meta) {
  if (bits < 2 || bits > 8 || !dims_ok(n, k) || k % kGroupSize != 0 || !meta_ok(meta)) return 0;
  return sizes_of(n, k, bits, kGroupSize, meta).zeros;
}

slq_status slq_quantize_pack(const float *W, int64_t n, int64_t k, int bits, int group,
                             slq_grid grid, slq_packed *out, slq_stream stream) {
  if (!out) return SLQ_EINVAL;
  if (bits < 2 || bits > 8) return SLQ_EINVAL;
  if (group <= 0) return SLQ_EINVAL;
  if (group != kGroupSize) return SLQ_ENOTSUP;
  if (grid != SLQ_ASYM && grid != SLQ_SYM) return SLQ_EINVAL;
  if (!dims_ok(n, k) || k % group != 0) return SLQ_EINVAL;
  if (!meta_ok(out->meta)) return SLQ_EINVAL;
  const PackedSizes sz = sizes_of(n, k, bits, group, out->meta);
  if (n * k > 0) {
    if (!W || !out->codes || !out->scales || !out->zeros) return SLQ_EINVAL;
    if (!aligned(W, 16) || !aligned(out->codes, 16) || !aligned(out->scales, 16) ||
        !aligned(out->zeros, 4))
      return SLQ_EINVAL;
    const size_t wb = (size_t)(n * k) * sizeof(float);
    if (overlap(W, wb, out->codes, sz.codes) || overlap(W, wb, out->scales, sz.scales) ||
        overlap(W, wb, out->zeros, sz.zeros) || overlap(out->codes, sz.codes, out->scales, sz.scales) ||
        overlap(out->codes, sz.codes, out->zeros, sz.zeros) ||
        overlap(out->scales, sz.scales, out->zeros, sz.zeros))
      return SLQ_EINVAL;
  }
  out->bits = bits;
  out->group = group;
  out->n = n;
  out->k = k;
  if (n * k == 0) return SLQ_OK;
  return from_hip(slq::launch_quantize_pack(W, n, k, bits, grid == SLQ_SYM,
                                            out->meta == SLQ_META_COMPACT, out->codes,
                                            out->scales, out->zeros,
                                            static_cast<hipStream_t>(stream)));
}

slq_status slq_dequantize(const slq_packed *w, float *W_deq, slq_stream stream) {
  PackedSizes sz;
  slq_status st = check_packed(w, &sz);
  if (st != SLQ_OK) return st;
  if (w->n * w->k == 0) return SLQ_OK;
  const size_t ob = (size_t)(w->n * w->k) * sizeof(float);
  if (!W_deq || !aligned(W_deq, 16)) return SLQ_EINVAL;
  if (overlap(W_deq, ob, w->codes, sz.codes) || overlap(W_deq, ob, w->scales, sz.scales) ||
      overlap(W_deq, ob, w->zeros, sz.zeros))
    return SLQ_EINVAL;
  return from_hip(slq::launch_dequantize(w->codes, w->scales, w->zeros,
                                         w->meta == SLQ_META_COMPACT, w->n, w->k, w->bits, W_deq,
                                         static_cast<hipStream_t>(stream)));
}

size_t slq_gemm_workspace_bytes(int64_t m, const slq_packed *w) {
  return gemm_ws_bytes(m, w);
}

}  // extern "C"

namespace {
size_t gemm_ws_bytes(int64_t m, const slq_packed *w) {
  PackedSizes sz;
  if (m < 0 || m >= kMaxDim || check_packed(w, &sz) != SLQ_OK) return 0;
  if (m == 0 || w->n == 0) return 0;
  if (m <= kDecodeMaxM) return slq::gemv_plan(m, w->n, w->k, w->bits).ws_bytes;
  return slq::gemm_workspace(m, w->n, w->k, w->bits);
}
}  // namespace

extern "C" {

slq_status slq_dequant_gemm(const uint16_t *x_bf16, const slq_packed *w, int64_t m, float *y,
                            void *workspace, slq_stream stream) {
  return dequant_gemm_checked(x_bf16, w, m, y, workspace, false, stream);
}

slq_status slq_dequant_gemm_noalloc(const uint16_t *x_bf16, const slq_packed *w, int64_t m,
                                    float *y, slq_stream stream) {
  return dequant_gemm_checked(x_bf16, w, m, y, nullptr, true, stream);
}

size_t slq_noalloc_scratch_bytes(void) { return kScratchBytes; }

const char *slq_dequant_gemm_kernel_name(int64_t m, const slq_packed *w) {
  static thread_local char buf[96];
  PackedSizes sz;
  buf[0] = '\0';
  if (m <= 0 || m >= kMaxDim || check_packed(w, &sz) != SLQ_OK) return buf;
  if (m <= kDecodeMaxM) {
    const slq::GemvPlan p = slq::gemv_plan(m, w->n, w->k, w->bits);
    const char *cm = w->meta == SLQ_META_COMPACT ? "true" : "false";
    if (p.tile)
      snprintf(buf, sizeof buf, "slq::gemv_tile_kernel<%d, %d, %d, %d, %s>", w->bits, p.mtw, p.ms, p.wv, cm);
    else if (p.mk)
      snprintf(buf, sizeof buf, "slq::gemv_mk_kernel<%d, %d, %d, %s>", w->bits, p.mt, p.nt, cm);
    else if (p.rows)
      snprintf(buf, sizeof buf, "slq::gemv_rows_kernel<%d, %d, %s>", w->bits, p.mt, cm);
    else
      snprintf(buf, sizeof buf, "slq::gemv_kernel<%d, %d, %d, %d, %s, %s, %d, %s>", w->bits, p.mt,
               p.nt, p.b, p.mv ? "true" : "false", p.xd ? "true" : "false", p.wv, cm);
  } else {
    snprintf(buf, sizeof buf, "slq::%s<%d, %s>",
             slq::gemm_plan(m, w->n, w->k).wide ? "gemm_wide_kernel" : "gemm_kernel", w->bits,
             w->meta == SLQ_META_COMPACT ? "true" : "false");
  }
  return buf;
}

size_t slq_ear_kl_workspace_bytes(int64_t rows, int64_t vocab) {
  if (rows < 0 || vocab < 0 || rows >= kMaxDim || vocab >= kMaxDim) return 0;
  return slq::fidelity_workspace(rows, vocab);
}

slq_status slq_row_lse(const float *logits, int64_t rows, int64_t vocab, double *lse,
                       void *workspace, slq_stream stream) {
  if (rows < 0 || vocab < 0 || rows >= kMaxDim || vocab >= kMaxDim) return SLQ_EINVAL;
  if (rows == 0) return SLQ_OK;
  if (vocab == 0) return SLQ_EINVAL;   // softmax over an empty vocabulary is undefined
  const size_t lb = (size_t)(rows * vocab) * sizeof(float);
  const size_t wsb = slq_ear_kl_workspace_bytes(rows, vocab);
  if (!logits || !lse || !workspace) return SLQ_EINVAL;
  if (!aligned(logits, 16) || !aligned(lse, 8) || !aligned(workspace, 256)) return SLQ_EINVAL;
  if (overlap(lse, rows * 8, logits, lb) || overlap(workspace, wsb, logits, lb) ||
      overlap(workspace, wsb, lse, rows * 8))
    return SLQ_EINVAL;
  return from_hip(slq::launch_row_lse(logits, rows, vocab, lse, workspace,
                                      static_cast<hipStream_t>(stream)));
}

namespace {

// Argument checks shared by the two EAR / KL entry points.
slq_status check_ear_kl(const float *logits_p, const float *logits_q, int64_t rows, int64_t vocab,
                        float *ear_rows, float *kl_rows, double *means, void *workspace) {
  const size_t lb = (size_t)(rows * vocab) * sizeof(float);
  const size_t rb = (size_t)rows * sizeof(float);
  const size_t wsb = slq_ear_kl_workspace_bytes(rows, vocab);
  if (!logits_p || !logits_q || !ear_rows || !kl_rows || !means || !workspace) return SLQ_EINVAL;
  if (!aligned(logits_p, 16) || !aligned(logits_q, 16) || !aligned(ear_rows, 4) ||
      !aligned(kl_rows, 4) || !aligned(means, 8) || !aligned(workspace, 256))
    return SLQ_EINVAL;
  const void *outs[4] = {ear_rows, kl_rows, means, workspace};
  const size_t outb[4] = {rb, rb, 2 * sizeof(double), wsb};
  for (int i = 0; i < 4; ++i) {
    if (overlap(outs[i], outb[i], logits_p, lb) || overlap(outs[i], outb[i], logits_q, lb))
      return SLQ_EINVAL;
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outb[i], outs[j], outb[j])) return SLQ_EINVAL;
  }
  return SLQ_OK;
}

}  // namespace

slq_status slq_ear_kl(const float *logits_p, const float *logits_q, int64_t rows, int64_t vocab,
                      float *ear_rows, float *kl_rows, double *means, void *workspace,
                      slq_stream stream) {
  if (rows < 0 || vocab < 0 || rows >= kMaxDim || vocab >= kMaxDim) return SLQ_EINVAL;
  if (rows == 0) return SLQ_OK;
  if (vocab == 0) return SLQ_EINVAL;
  const slq_status st =
      check_ear_kl(logits_p, logits_q, rows, vocab, ear_rows, kl_rows, means, workspace);
  if (st != SLQ_OK) return st;
  return from_hip(slq::launch_ear_kl(logits_p, logits_q, rows, vocab, ear_rows, kl_rows, means,
                                     workspace, static_cast<hipStream_t>(stream)));
}

slq_status slq_ear_kl_topk(const float *logits_p, const float *logits_q, int64_t rows,
                           int64_t vocab, int64_t K, double temperature, float *ear_rows,
                           float *kl_rows, double *means, void *workspace, slq_stream stream) {
  static_assert(SLQ_TOPK_MAX == slq::kTopKMax, "top-K limit of the header and the kernels");
  if (rows < 0 || vocab < 0 || rows >= kMaxDim || vocab >= kMaxDim) return SLQ_EINVAL;
  if (K < 1 || K > SLQ_TOPK_MAX || (vocab > 0 && K > vocab)) return SLQ_EINVAL;
  if (!(temperature > 0.0) || !std::isfinite(temperature)) return SLQ_EINVAL;
  const double invT = 1.0 / temperature;
  // the fp32 exponent scale log2(e) / T must be finite and nonzero
  const float c = (float)(1.4426950408889634 * invT);
  if (!(c > 0.0f) || !std::isfinite(c)) return SLQ_EINVAL;
  if (rows == 0) return SLQ_OK;
  if (vocab == 0) return SLQ_EINVAL;
  const slq_status st =
      check_ear_kl(logits_p, logits_q, rows, vocab, ear_rows, kl_rows, means, workspace);
  if (st != SLQ_OK) return st;
  return from_hip(slq::launch_ear_kl_topk(logits_p, logits_q, rows, vocab, (int)K, invT, ear_rows,
                                          kl_rows, means, workspace,
                                          static_cast<hipStream_t>(stream)));
}

size_t slq_gptq_workspace_bytes(int64_t n, int64_t k) {
  if (n < 1 || n >= kMaxDim || k < kGroupSize || k > 32768 || k % kGroupSize != 0) return 0;
  return slq::gptq_workspace(n, k);
}

slq_status slq_gptq_quantize(const float *W, const float *H, int64_t n, int64_t k, int bits,
                             int group, double damp, slq_packed *out, double *u_out,
                             void *workspace, slq_stream stream) {
  if (!out || bits < 2 || bits > 8 || group <= 0) return SLQ_EINVAL;
  if (group != kGroupSize) return SLQ_ENOTSUP;
  if (n < 1 || n >= kMaxDim || k < kGroupSize || k > 32768 || k % kGroupSize != 0 ||
      n * k >= kMaxDim * 64)
    return SLQ_EINVAL;
  if (!(damp > 0.0) || !std::isfinite(damp)) return SLQ_EINVAL;
  if (!meta_ok(out->meta)) return SLQ_EINVAL;
  if (out->meta != SLQ_META_F32) return SLQ_ENOTSUP;
  const PackedSizes sz = sizes_of(n, k, bits, group, out->meta);
  const size_t wsb = slq_gptq_workspace_bytes(n, k);
  if (!W || !H || !workspace || !out->codes || !out->scales || !out->zeros) return SLQ_EINVAL;
  if (!aligned(W, 16) || !aligned(H, 16) || !aligned(workspace, 256) || !aligned(out->codes, 16) ||
      !aligned(out->scales, 16) || !aligned(out->zeros, 4) || (u_out && !aligned(u_out, 8)))
    return SLQ_EINVAL;
  const size_t wb = (size_t)(n * k) * 4, hb = (size_t)(k * k) * 4, ub = (size_t)(k * k) * 8;
  const void *in[2] = {W, H};
  const size_t inb[2] = {wb, hb};
  const void *outs[5] = {out->codes, out->scales, out->zeros, workspace, u_out};
  const size_t outb[5] = {sz.codes, sz.scales, sz.zeros, wsb, u_out ? ub : 0};
  for (int i = 0; i < 5; ++i) {
    if (!outs[i]) continue;
    for (int j = 0; j < 2; ++j)
      if (overlap(outs[i], outb[i], in[j], inb[j])) return SLQ_EINVAL;
    for (int j = i + 1; j < 5; ++j)
      if (outs[j] && overlap(outs[i], outb[i], outs[j], outb[j])) return SLQ_EINVAL;
  }
  out->bits = bits;
  out->group = group;
  out->n = n;
  out->k = k;
  return from_hip(slq::launch_gptq(W, H, n, k, bits, damp, out->codes,
                                   static_cast<float *>(out->scales), out->zeros, u_out, workspace,
                                   static_cast<hipStream_t>(stream)));
}

static bool gptq_k_ok(int64_t k) { return k >= kGroupSize && k <= 32768 && k % kGroupSize == 0; }

size_t slq_gptq_factor_workspace_bytes(int64_t k) {
  if (!gptq_k_ok(k)) return 0;
  return slq::gptq_factor_workspace(k);
}

slq_status slq_gptq_factor(const float *H, int64_t k, double damp, float *U, uint8_t *dead,
                           double *u_out, void *workspace, slq_stream stream) {
  if (!gptq_k_ok(k) || !(damp > 0.0) || !std::isfinite(damp)) return SLQ_EINVAL;
  if (!H || !U || !dead || !workspace) return SLQ_EINVAL;
  if (!aligned(H, 16) || !aligned(U, 16) || !aligned(workspace, 256) || (u_out && !aligned(u_out, 8)))
    return SLQ_EINVAL;
  const size_t hb = (size_t)(k * k) * 4;
  const void *outs[4] = {U, dead, u_out, workspace};
  const size_t outb[4] = {(size_t)(k * k) * 4, (size_t)k, u_out ? (size_t)(k * k) * 8 : 0,
                          slq_gptq_factor_workspace_bytes(k)};
  for (int i = 0; i < 4; ++i) {
    if (!outs[i]) continue;
    if (overlap(outs[i], outb[i], H, hb)) return SLQ_EINVAL;
    for (int j = i + 1; j < 4; ++j)
      if (outs[j] && overlap(outs[i], outb[i], outs[j], outb[j])) return SLQ_EINVAL;
  }
  return from_hip(slq::launch_gptq_factor(H, k, damp, U, dead, u_out, workspace,
                                          static_cast<hipStream_t>(stream)));
}

size_t slq_gptq_columns_workspace_bytes(int64_t n, int64_t k) {
  if (n < 1 || n >= kMaxDim || !gptq_k_ok(k) || n * k >= kMaxDim * 64) return 0;
  return slq::gptq_columns_workspace(n, k);
}

slq_status slq_gptq_columns(const float *W, const float *U, const uint8_t *dead, int64_t n,
                            int64_t k, int bits, int group, slq_packed *out, void *workspace,
                            slq_stream stream) {
  if (!out || bits < 2 || bits > 8 || group <= 0) return SLQ_EINVAL;
  if (group != kGroupSize) return SLQ_ENOTSUP;
  if (n < 1 || n >= kMaxDim || !gptq_k_ok(k) || n * k >= kMaxDim * 64) return SLQ_EINVAL;
  if (!meta_ok(out->meta)) return SLQ_EINVAL;
  if (out->meta != SLQ_META_F32) return SLQ_ENOTSUP;
  if (!W || !U || !workspace || !out->codes || !out->scales || !out->zeros) return SLQ_EINVAL;
  if (!aligned(W, 16) || !aligned(U, 16) || !aligned(workspace, 256) || !aligned(out->codes, 16) ||
      !aligned(out->scales, 16) || !aligned(out->zeros, 4))
    return SLQ_EINVAL;
  const PackedSizes sz = sizes_of(n, k, bits, group, out->meta);
  const void *in[3] = {W, U, dead};
  const size_t inb[3] = {(size_t)(n * k) * 4, (size_t)(k * k) * 4, dead ? (size_t)k : 0};
  const void *outs[4] = {out->codes, out->scales, out->zeros, workspace};
  const size_t outb[4] = {sz.codes, sz.scales, sz.zeros, slq_gptq_columns_workspace_bytes(n, k)};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 3; ++j)
      if (in[j] && overlap(outs[i], outb[i], in[j], inb[j])) return SLQ_EINVAL;
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outb[i], outs[j], outb[j])) return SLQ_EINVAL;
  }
  out->bits = bits;
  out->group = group;
  out->n = n;
  out->k = k;
  return from_hip(slq::launch_gptq_columns(W, U, dead, n, k, bits, out->codes,
                                           static_cast<float *>(out->scales), out->zeros,
                                           workspace, static_cast<hipStream_t>(stream)));
}

size_t slq_mckp_workspace_bytes(int64_t L, int64_t W) {
  if (L < 1 || L >= kMaxDim || W < 0 || W >= kMaxDim - 1) return 0;
  return slq::mckp_workspace(L, W);
}

slq_status slq_mckp_search(const int64_t *sizes, const double *costs, int64_t L, int32_t nb,
                           int64_t W, double tau, int32_t *choice, int64_t *result, double *cost,
                           double *best, void *workspace, slq_stream stream) {
  if (L < 1 || L >= kMaxDim || nb < 1 || nb > 127 || W < 0 || W >= kMaxDim - 1) return SLQ_EINVAL;
  if (std::isnan(tau)) return SLQ_EINVAL;
  if (!sizes || !costs || !choice || !result || !cost || !workspace) return SLQ_EINVAL;
  if (!aligned(sizes, 8) || !aligned(costs, 8) || !aligned(choice, 4) || !aligned(result, 8) ||
      !aligned(cost, 8) || !aligned(workspace, 256) || (best && !aligned(best, 8)))
    return SLQ_EINVAL;
  const size_t tb = (size_t)L * nb * 8;
  const size_t wsb = slq_mckp_workspace_bytes(L, W);
  const void *outs[5] = {choice, result, cost, workspace, best};
  const size_t outb[5] = {(size_t)L * 4, 3 * sizeof(int64_t), sizeof(double), wsb,
                          best ? (size_t)(W + 1) * sizeof(double) : 0};
  for (int i = 0; i < 5; ++i) {
    if (!outs[i]) continue;
    if (overlap(outs[i], outb[i], sizes, tb) || overlap(outs[i], outb[i], costs, tb))
      return SLQ_EINVAL;
    for (int j = i + 1; j < 5; ++j)
      if (outs[j] && overlap(outs[i], outb[i], outs[j], outb[j])) return SLQ_EINVAL;
  }
  return from_hip(slq::launch_mckp(sizes, costs, L, nb, W, tau, choice, result, cost, best,
                                   workspace, static_cast<hipStream_t>(stream)));
}

size_t slq_quant_error_workspace_bytes(const slq_packed *w) {
  PackedSizes sz;
  if (check_packed(w, &sz) != SLQ_OK) return 0;
  return slq::quant_error_workspace(w->n, w->k);
}

slq_status slq_quant_error(const float *W, const slq_packed *w, double *out, void *workspace,
                           slq_stream stream) {
  PackedSizes sz;
  slq_status st = check_packed(w, &sz);
  if (st != SLQ_OK) return st;
  if (!out || !aligned(out, 8)) return SLQ_EINVAL;
  const size_t wb = (size_t)(w->n * w->k) * sizeof(float);
  const size_t wsb = slq_quant_error_workspace_bytes(w);
  if (wb > 0 && (!W || !aligned(W, 16))) return SLQ_EINVAL;
  if (wsb > 0 && (!workspace || !aligned(workspace, 256))) return SLQ_EINVAL;
  if (overlap(out, 16, W, wb) || overlap(out, 16, workspace, wsb) ||
      overlap(workspace, wsb, W, wb) || overlap(out, 16, w->codes, sz.codes) ||
      overlap(out, 16, w->scales, sz.scales) || overlap(out, 16, w->zeros, sz.zeros) ||
      overlap(workspace, wsb, w->codes, sz.codes) || overlap(workspace, wsb, w->scales, sz.scales) ||
      overlap(workspace, wsb, w->zeros, sz.zeros))
    return SLQ_EINVAL;
  return from_hip(slq::launch_quant_error(W, w->codes, w->scales, w->zeros,
                                          w->meta == SLQ_META_COMPACT, w->n, w->k, w->bits, out,
                                          workspace, static_cast<hipStream_t>(stream)));
}

size_t slq_stream_read_words(size_t bytes) { return slq::stream_read_words(bytes); }

slq_status slq_stream_read(const void *buf, size_t bytes, uint32_t *folds, slq_stream stream) {
  if (bytes == 0) return SLQ_OK;
  if (!buf || !folds || bytes % 16 != 0 || !aligned(buf, 16) || !aligned(folds, 4)) return SLQ_EINVAL;
  if (overlap(buf, bytes, folds, slq_stream_read_words(bytes) * 4)) return SLQ_EINVAL;
  return from_hip(slq::launch_stream_read(buf, bytes, folds, static_cast<hipStream_t>(stream)));
}

const char *slq_strerror(slq_status s) {
  switch (s) {
    case SLQ_OK: return "ok";
    case SLQ_EINVAL: return "invalid argument (size, bit-width, pointer, alignment or aliasing)";
    case SLQ_ENOTSUP: return "unsupported request (group size other than 128)";
    case SLQ_EHIP: return "HIP runtime error at launch";
    case SLQ_ESCRATCH:
      return "the request needs more split-k scratch than the allocation-free entry point holds";
  }
  return "unknown status";
}

}  // extern "C"
