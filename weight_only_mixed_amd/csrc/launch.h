// Internal launchers behind the C ABI (host code; arguments already validated).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace slq {

// quantize.hip
// `compact`: binary16 scales and nibble (b <= 4) or byte zero points; else
// fp32 scales and byte zero points.
hipError_t launch_quantize_pack(const float *W, int64_t n, int64_t k, int bits, bool symmetric,
                                bool compact, uint32_t *codes, void *scales, uint8_t *zeros,
                                hipStream_t s);
hipError_t launch_dequantize(const uint32_t *codes, const void *scales, const uint8_t *zeros,
                             bool compact, int64_t n, int64_t k, int bits, float *out,
                             hipStream_t s);
size_t quant_error_workspace(int64_t n, int64_t k);
hipError_t launch_quant_error(const float *W, const uint32_t *codes, const void *scales,
                              const uint8_t *zeros, bool compact, int64_t n, int64_t k, int bits,
                              double *out, void *ws, hipStream_t s);

// gemv.hip (decode, m <= 64)
struct GemvPlan {
  int mt;          // 16-row tiles of x
  int nt;          // 16-row weight tiles per workgroup
  int wv;          // wavefronts per workgroup (all on the same rows, splitting k)
  int b;           // groups per load batch
  int gw;          // 128-groups per k-block (workgroup)
  int nblocks;     // workgroups along n
  int ksplits;     // workgroups along k (0: shape not supported)
  bool mv;         // scales/zero points staged as vectors of 4 groups per row
  bool xd;         // activations loaded by each lane with the weight batches (mt == 1)
  bool rows;       // 17..64 activation rows: row-split kernel, 64 rows per workgroup
  bool mk;         // 33..64 activation rows, mid-width layer: gemv_mk_kernel, 64 * nt rows per workgroup
  bool tile;       // 17..64 activation rows: gemv_tile_kernel, 16 * nt rows per workgroup
  int ms;          // tile kernel: wavefronts along the activation rows (the rest split k)
  int mtw;         // tile kernel: 16-row activation tiles per wavefront
  size_t ws_bytes; // tickets + partial sums
};
GemvPlan gemv_plan(int64_t m, int64_t n, int64_t k, int bits);
hipError_t launch_gemv(const uint16_t *x, const uint32_t *codes, const void *scales,
                       const uint8_t *zeros, bool compact, int64_t m, int64_t n, int64_t k,
                       int bits, float *y, void *ws, const GemvPlan &plan, hipStream_t s);

// gemm.hip (prefill, m > 64)
size_t gemm_workspace(int64_t m, int64_t n, int64_t k, int bits);
struct GemmPlan {
  bool wide;    // gemm_wide_kernel (256 x 256 tiles) rather than gemm_kernel
  int split;    // k splits (partial tiles in the workspace, summed in order)
  int ksteps;   // 64-wide k steps per split
};
GemmPlan gemm_plan(int64_t m, int64_t n, int64_t k);
hipError_t launch_gemm(const uint16_t *x, const uint32_t *codes, const void *scales,
                       const uint8_t *zeros, bool compact, int64_t m, int64_t n, int64_t k,
                       int bits, float *y, void *ws, hipStream_t s);

// fidelity.hip
size_t fidelity_workspace(int64_t rows, int64_t vocab);
hipError_t launch_row_lse(const float *a, int64_t rows, int64_t vocab, double *lse, void *ws,
                          hipStream_t s);
hipError_t launch_ear_kl(const float *a, const float *b, int64_t rows, int64_t vocab, float *ear,
                         float *kl, double *means, void *ws, hipStream_t s);
size_t gptq_workspace(int64_t n, int64_t k);
size_t gptq_factor_workspace(int64_t k);
size_t gptq_columns_workspace(int64_t n, int64_t k);
// U fp32 [k][k] upper with U^T U = (H + damping)^-1, dead [k] = (H_ii == 0)
hipError_t launch_gptq_factor(const float *H, int64_t k, double damp, float *Uf, uint8_t *dead,
                              double *u_out, void *ws, hipStream_t s);
hipError_t launch_gptq_columns(const float *W, const float *Uf, const uint8_t *dead, int64_t n,
                               int64_t k, int bits, uint32_t *codes, float *scales,
                               uint8_t *zeros, void *ws, hipStream_t s);
hipError_t launch_gptq(const float *W, const float *H, int64_t n, int64_t k, int bits, double damp,
                       uint32_t *codes, float *scales, uint8_t *zeros, double *u_out, void *ws,
                       hipStream_t s);
size_t mckp_workspace(int64_t L, int64_t W);
hipError_t launch_mckp(const int64_t *sizes, const double *costs, int64_t L, int nb, int64_t W,
                       double tau, int32_t *choice, int64_t *result, double *cost, double *best,
                       void *ws, hipStream_t s);
constexpr int kTopKMax = 64;   // largest k of the top-K metrics
// invT = 1 / temperature.
hipError_t launch_ear_kl_topk(const float *a, const float *b, int64_t rows, int64_t vocab, int k,
                              double invT, float *ear, float *kl, double *means, void *ws,
                              hipStream_t s);

// noalloc.hip: the split-k scratch of the allocation-free matmul, a static
// device array per GPU; its device address for the current device
constexpr size_t kNoallocScratchBytes = (size_t)32 << 20;
hipError_t noalloc_scratch(void **out, hipStream_t s);

// probe.hip: one plain read of `bytes` (a multiple of 16) of `buf`; one XOR
// fold per 16 KiB read into folds[stream_read_words(bytes)]
size_t stream_read_words(size_t bytes);
hipError_t launch_stream_read(const void *buf, size_t bytes, uint32_t *folds, hipStream_t s);

}  // namespace slq
