// Drives every entry point of the C ABI through its validation (invalid
// arguments, empty sizes, and valid requests that reach a launcher that
// reports an error), under AddressSanitizer and UndefinedBehaviorSanitizer.
// Pointers are fake device addresses that validation never dereferences.
#include <stdint.h>
#include <stdio.h>

#include "../../include/slq.h"

static int fails = 0;
#define EXPECT(call, want)                                                              \
  do {                                                                                  \
    const int got_ = (int)(call);                                                       \
    if (got_ != (int)(want)) {                                                          \
      fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__, #call, got_, \
              (int)(want));                                                             \
      ++fails;                                                                          \
    }                                                                                   \
  } while (0)

static void *P(uintptr_t a) { return reinterpret_cast<void *>(a); }

int main() {
  const uintptr_t A = 0x10000000, B = 0x20000000, C = 0x30000000, D = 0x40000000, E = 0x50000000;
  slq_packed w{4, 128, 64, 256, (uint32_t *)P(B), P(C), (uint8_t *)P(D), SLQ_META_F32, 0};
  slq_packed out{0, 0, 0, 0, (uint32_t *)P(B), P(C), (uint8_t *)P(D), SLQ_META_F32, 0};
  // quantize / pack
  EXPECT(slq_quantize_pack((const float *)P(A), 64, 256, 1, 128, SLQ_ASYM, &out, nullptr), SLQ_EINVAL);
  EXPECT(slq_quantize_pack((const float *)P(A), 64, 256, 4, 64, SLQ_ASYM, &out, nullptr), SLQ_ENOTSUP);
  EXPECT(slq_quantize_pack((const float *)P(A), 64, 200, 4, 128, SLQ_ASYM, &out, nullptr), SLQ_EINVAL);
  EXPECT(slq_quantize_pack((const float *)P(A + 4), 64, 256, 4, 128, SLQ_ASYM, &out, nullptr), SLQ_EINVAL);
  EXPECT(slq_quantize_pack((const float *)P(A), 0, 256, 4, 128, SLQ_ASYM, &out, nullptr), SLQ_OK);
  EXPECT(slq_quantize_pack((const float *)P(A), 64, 256, 4, 128, SLQ_ASYM, &out, nullptr), SLQ_EHIP);
  EXPECT(slq_quantize_pack((const float *)P(A), INT64_MAX, 256, 4, 128, SLQ_ASYM, &out, nullptr), SLQ_EINVAL);
  EXPECT(slq_codes_bytes(64, 256, 3), 64 * 256 * 3 / 8);
  EXPECT(slq_codes_bytes(-1, 256, 3), 0);
  EXPECT(slq_scales_bytes(INT64_MAX, 128, SLQ_META_F32), 0);
  // dequantize and the matmul
  EXPECT(slq_dequantize(&w, (float *)P(E), nullptr), SLQ_EHIP);
  EXPECT(slq_dequantize(&w, (float *)P(B), nullptr), SLQ_EINVAL);              // overlaps codes
  EXPECT(slq_dequant_gemm((const uint16_t *)P(A), &w, 1, (float *)P(E), nullptr, nullptr), SLQ_EHIP);
  EXPECT(slq_dequant_gemm((const uint16_t *)P(A), &w, 100, (float *)P(E), nullptr, nullptr), SLQ_EHIP);
  EXPECT(slq_dequant_gemm((const uint16_t *)P(A), &w, -1, (float *)P(E), nullptr, nullptr), SLQ_EINVAL);
  EXPECT(slq_dequant_gemm((const uint16_t *)P(A), &w, 0, (float *)P(E), nullptr, nullptr), SLQ_OK);
  EXPECT(slq_dequant_gemm((const uint16_t *)P(A), &w, 1, (float *)P(A), nullptr, nullptr), SLQ_EINVAL);
  EXPECT(slq_dequant_gemm(nullptr, &w, 1, (float *)P(E), nullptr, nullptr), SLQ_EINVAL);
  EXPECT(slq_dequant_gemm((const uint16_t *)P(A), nullptr, 1, (float *)P(E), nullptr, nullptr), SLQ_EINVAL);
  (void)slq_dequant_gemm_kernel_name(1, &w);
  (void)slq_dequant_gemm_kernel_name(-5, nullptr);
  (void)slq_gemm_workspace_bytes(64, &w);
  // fidelity
  EXPECT(slq_row_lse((const float *)P(A), 4, 100, (double *)P(B), P(E), nullptr), SLQ_EHIP);
  EXPECT(slq_row_lse((const float *)P(A), 4, 0, (double *)P(B), P(E), nullptr), SLQ_EINVAL);
  EXPECT(slq_ear_kl((const float *)P(A), (const float *)P(B), 4, 100, (float *)P(C), (float *)P(C + 64),
                    (double *)P(D), P(E), nullptr), SLQ_EHIP);
  EXPECT(slq_ear_kl((const float *)P(A), (const float *)P(A), 4, 100, (float *)P(A), (float *)P(C + 64),
                    (double *)P(D), P(E), nullptr), SLQ_EINVAL);
  EXPECT(slq_ear_kl_topk((const float *)P(A), (const float *)P(B), 4, 100, 10, 1.0, (float *)P(C),
                         (float *)P(C + 64), (double *)P(D), P(E), nullptr), SLQ_EHIP);
  EXPECT(slq_ear_kl_topk((const float *)P(A), (const float *)P(B), 4, 100, 0, 1.0, (float *)P(C),
                         (float *)P(C + 64), (double *)P(D), P(E), nullptr), SLQ_EINVAL);
  EXPECT(slq_ear_kl_topk((const float *)P(A), (const float *)P(B), 4, 100, 10, 1e-300, (float *)P(C),
                         (float *)P(C + 64), (double *)P(D), P(E), nullptr), SLQ_EINVAL);
  (void)slq_ear_kl_workspace_bytes(INT64_MAX, INT64_MAX);
  // GPTQ
  slq_packed g{0, 0, 0, 0, (uint32_t *)P(C), P(C + 0x100000), (uint8_t *)P(C + 0x200000), SLQ_META_F32, 0};
  EXPECT(slq_gptq_quantize((const float *)P(A), (const float *)P(B), 64, 256, 4, 128, 0.01, &g, nullptr,
                           P(E), nullptr), SLQ_EHIP);
  EXPECT(slq_gptq_quantize((const float *)P(A), (const float *)P(B), 64, 256, 4, 128, 0.0, &g, nullptr,
                           P(E), nullptr), SLQ_EINVAL);
  EXPECT(slq_gptq_factor((const float *)P(A), 256, 0.01, (float *)P(B), (uint8_t *)P(C), nullptr, P(E),
                         nullptr), SLQ_EHIP);
  EXPECT(slq_gptq_factor((const float *)P(A), 200, 0.01, (float *)P(B), (uint8_t *)P(C), nullptr, P(E),
                         nullptr), SLQ_EINVAL);
  EXPECT(slq_gptq_columns((const float *)P(A), (const float *)P(B), nullptr, 64, 256, 4, 128, &g, P(E),
                          nullptr), SLQ_EHIP);
  EXPECT(slq_gptq_columns((const float *)P(A), (const float *)P(B), (const uint8_t *)P(C + 0x100000 + 8),
                          64, 256, 4, 128, &g, P(E), nullptr), SLQ_EINVAL);
  (void)slq_gptq_workspace_bytes(64, 256);
  (void)slq_gptq_factor_workspace_bytes(INT64_MAX);
  (void)slq_gptq_columns_workspace_bytes(INT64_MAX, 256);
  // allocation
  EXPECT(slq_mckp_search((const int64_t *)P(A), (const double *)P(B), 4, 7, 100, 1.0, (int32_t *)P(C),
                         (int64_t *)P(C + 256), (double *)P(C + 512), nullptr, P(E), nullptr), SLQ_EHIP);
  EXPECT(slq_mckp_search((const int64_t *)P(A), (const double *)P(B), 4, 128, 100, 1.0, (int32_t *)P(C),
                         (int64_t *)P(C + 256), (double *)P(C + 512), nullptr, P(E), nullptr), SLQ_EINVAL);
  (void)slq_mckp_workspace_bytes(INT64_MAX, INT64_MAX);
  // noise sums, the read probe, status strings
  EXPECT(slq_quant_error((const float *)P(A), &w, (double *)P(E), P(E + 0x1000), nullptr), SLQ_EHIP);
  EXPECT(slq_quant_error((const float *)P(A), nullptr, (double *)P(E), P(E + 0x1000), nullptr), SLQ_EINVAL);
  (void)slq_quant_error_workspace_bytes(&w);
  EXPECT(slq_stream_read(P(A), 4096, (uint32_t *)P(B), nullptr), SLQ_EHIP);
  EXPECT(slq_stream_read(P(A), 4097, (uint32_t *)P(B), nullptr), SLQ_EINVAL);
  for (int s = -1; s < 6; ++s) (void)slq_strerror((slq_status)s);
  printf("abi sanitizer driver: %d failing checks\n", fails);
  return fails ? 1 : 0;
}
