// Split-k scratch of the allocation-free matmul (slq_dequant_gemm_noalloc):
// one static device array per GPU, held until the process ends.  In host code
// `scratch` is only a stand-in for the device array, so its device address is
// looked up with hipGetSymbolAddress, once per device with that device
// current, and only that address is handed to the kernels.
#include <mutex>

#include "launch.h"

namespace slq {
namespace {

__device__ __attribute__((aligned(256))) unsigned char scratch[kNoallocScratchBytes];

constexpr size_t kTicketArea = 65536;   // decode split-k tickets, kept zero between calls
constexpr int kMaxDevices = 64;
void *g_ptr[kMaxDevices];
hipError_t g_status[kMaxDevices];
std::once_flag g_once[kMaxDevices];

__global__ void zero_words_kernel(uint32_t *__restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

}  // namespace

// The current device's scratch address.  The first call on a device looks it
// up and clears the ticket area with a fill kernel on `s` (a memset node would
// be unsafe under graph capture); later calls find the tickets at zero, since
// every completed call leaves them so.
hipError_t noalloc_scratch(void **out, hipStream_t s) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_once[dev], [&] {
    void *p = nullptr;
    hipError_t r = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (r == hipSuccess) {
      hipLaunchKernelGGL(zero_words_kernel, dim3(64), dim3(256), 0, s, static_cast<uint32_t *>(p),
                         (int64_t)(kTicketArea / 4));
      r = hipGetLastError();
    }
    g_ptr[dev] = r == hipSuccess ? p : nullptr;
    g_status[dev] = r;
  });
  *out = g_ptr[dev];
  return g_status[dev];
}

}  // namespace slq
