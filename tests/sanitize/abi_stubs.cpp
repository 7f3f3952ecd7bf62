// Host-only stand-ins for the kernel launchers behind the C ABI, so that the
// argument validation of slq_abi.cpp can be built with g++ under
// AddressSanitizer and UndefinedBehaviorSanitizer and driven on a machine with
// no GPU.  Every launcher reports an error; the plans describe a one-split
// decode with a small workspace.
#include "../../weight_only_mixed_amd/csrc/launch.h"

namespace slq {
hipError_t launch_quantize_pack(const float *, int64_t, int64_t, int, bool, bool, uint32_t *, void *,
                                uint8_t *, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_dequantize(const uint32_t *, const void *, const uint8_t *, bool, int64_t, int64_t,
                             int, float *, hipStream_t) { return hipErrorInvalidValue; }
size_t quant_error_workspace(int64_t n, int64_t k) { return (size_t)(n * (k / 32)) * 16 + 16; }
hipError_t launch_quant_error(const float *, const uint32_t *, const void *, const uint8_t *, bool,
                              int64_t, int64_t, int, double *, void *, hipStream_t) {
  return hipErrorInvalidValue;
}
GemvPlan gemv_plan(int64_t m, int64_t, int64_t, int) {
  GemvPlan p{};
  p.mt = (int)((m + 15) / 16);
  p.nt = 1;
  p.wv = 4;
  p.b = 1;
  p.gw = 1;
  p.nblocks = 1;
  p.ksplits = 1;
  p.ws_bytes = 0;
  return p;
}
hipError_t launch_gemv(const uint16_t *, const uint32_t *, const void *, const uint8_t *, bool,
                       int64_t, int64_t, int64_t, int, float *, void *, const GemvPlan &,
                       hipStream_t) { return hipErrorInvalidValue; }
size_t gemm_workspace(int64_t, int64_t, int64_t, int) { return 0; }
GemmPlan gemm_plan(int64_t, int64_t, int64_t) { return GemmPlan{true, 1, 1}; }
hipError_t launch_gemm(const uint16_t *, const uint32_t *, const void *, const uint8_t *, bool,
                       int64_t, int64_t, int64_t, int, float *, void *, hipStream_t) {
  return hipErrorInvalidValue;
}
size_t fidelity_workspace(int64_t rows, int64_t) { return (size_t)rows * 64 + 256; }
hipError_t launch_row_lse(const float *, int64_t, int64_t, double *, void *, hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t launch_ear_kl(const float *, const float *, int64_t, int64_t, float *, float *, double *,
                         void *, hipStream_t) { return hipErrorInvalidValue; }
size_t gptq_workspace(int64_t n, int64_t k) { return (size_t)(n * k + k * k) * 4 + 256; }
size_t gptq_factor_workspace(int64_t k) { return (size_t)k * k * 16 + 256; }
size_t gptq_columns_workspace(int64_t n, int64_t k) { return (size_t)(n * k + n * 128) * 4; }
hipError_t launch_gptq_factor(const float *, int64_t, double, float *, uint8_t *, double *, void *,
                              hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_gptq_columns(const float *, const float *, const uint8_t *, int64_t, int64_t, int,
                               uint32_t *, float *, uint8_t *, void *, hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t launch_gptq(const float *, const float *, int64_t, int64_t, int, double, uint32_t *,
                       float *, uint8_t *, double *, void *, hipStream_t) {
  return hipErrorInvalidValue;
}
size_t mckp_workspace(int64_t L, int64_t W) { return (size_t)(L * (W + 1)) + (size_t)(W + 1) * 16; }
hipError_t launch_mckp(const int64_t *, const double *, int64_t, int, int64_t, double, int32_t *,
                       int64_t *, double *, double *, void *, hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t launch_ear_kl_topk(const float *, const float *, int64_t, int64_t, int, double, float *,
                              float *, double *, void *, hipStream_t) { return hipErrorInvalidValue; }
hipError_t noalloc_scratch(void **out, hipStream_t) {
  *out = nullptr;
  return hipErrorInvalidValue;
}
size_t stream_read_words(size_t bytes) { return (bytes + 16383) / 16384; }
hipError_t launch_stream_read(const void *, size_t, uint32_t *, hipStream_t) {
  return hipErrorInvalidValue;
}
}  // namespace slq
