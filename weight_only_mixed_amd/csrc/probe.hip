// Plain read of a device buffer, for calibrating the HBM read ceiling and the
// per-launch floor against which the decode kernels are judged: every
// workgroup reads 256 x kUnroll consecutive 16-byte words with coalesced
// 16-byte loads, folds them with XOR and writes its fold to its own word of
// `folds`, so the reads cannot be dropped and no two workgroups contend.
#include "launch.h"
#include "slq_device.h"

namespace slq {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4_t *__restrict__ p,
                                                               int64_t n16,
                                                               uint32_t *__restrict__ folds) {
  __shared__ uint32_t wf[kThreads / kWave];
  const int64_t base = (int64_t)blockIdx.x * kThreads * kUnroll + threadIdx.x;
  u32x4_t v[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int64_t i = base + (int64_t)u * kThreads;
    v[u] = i < n16 ? p[i] : u32x4_t{0u, 0u, 0u, 0u};
  }
  uint32_t f = 0u;
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) f ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) f ^= __shfl_xor(f, o, kWave);
  if ((threadIdx.x & (kWave - 1)) == 0) wf[threadIdx.x / kWave] = f;
  __syncthreads();
  if (threadIdx.x == 0) folds[blockIdx.x] = wf[0] ^ wf[1] ^ wf[2] ^ wf[3];
}

}  // namespace

size_t stream_read_words(size_t bytes) {
  const size_t per = (size_t)kThreads * kUnroll * 16;
  return (bytes + per - 1) / per;
}

hipError_t launch_stream_read(const void *buf, size_t bytes, uint32_t *folds, hipStream_t s) {
  const int64_t n16 = (int64_t)(bytes / 16);
  if (n16 == 0) return hipSuccess;
  const int64_t per = (int64_t)kThreads * kUnroll;
  const int64_t blocks = (n16 + per - 1) / per;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s,
                     static_cast<const u32x4_t *>(buf), n16, folds);
  return hipGetLastError();
}

}  // namespace slq
