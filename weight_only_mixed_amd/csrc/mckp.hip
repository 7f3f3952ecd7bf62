// Bit-width allocation for gfx950: exact multiple-choice knapsack over a cost
// table for every budget, then the smallest budget that meets a target
// (gist.science summary "Statistically-Lossless Quantization of Large
// Language Models", 3. The SLQ Pipeline: allocation as a multiple-choice
// knapsack solved exactly under a bit budget; SLQ README, Pipeline: the budget
// is found by bisection until the target is met).
//
// Item l takes one of nb options; option j occupies s_lj budget units and
// costs c_lj.  best_l(w) = least cost of items 0..l within budget w:
//   best_{-1}(w) = 0,  best_l(w) = min_j best_{l-1}(w - s_lj) + c_lj  (s_lj <= w),
// ties to the lower j.  One launch per item updates every budget in parallel
// (the items are a chain, the budgets are independent); the option taken at
// every (l, w) is kept for the read-back.  A last single-lane kernel finds the
// smallest budget whose best cost is finite and <= tau by binary search
// (best is non-increasing in w) and walks the choices back from the last item.
#include <cmath>

#include "launch.h"

namespace slq {
namespace {

constexpr int kMckpThreads = 256;

__global__ __launch_bounds__(kMckpThreads) void mckp_zero_kernel(double *__restrict__ row,
                                                                 int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * kMckpThreads + threadIdx.x;
  if (i < n) row[i] = 0.0;
}

__global__ __launch_bounds__(kMckpThreads) void mckp_item_kernel(
    const int64_t *__restrict__ sizes, const double *__restrict__ costs, int nb, int64_t item,
    int64_t W, const double *__restrict__ prev, double *__restrict__ cur,
    int8_t *__restrict__ pick) {
  const int64_t w = (int64_t)blockIdx.x * kMckpThreads + threadIdx.x;
  if (w > W) return;
  double b = INFINITY;
  int jb = -1;
  for (int j = 0; j < nb; ++j) {
    const int64_t sz = sizes[item * nb + j];
    if (sz < 0 || sz > w) continue;   // negative sizes: never selectable
    const double v = prev[w - sz] + costs[item * nb + j];
    if (v < b) {
      b = v;
      jb = j;
    }
  }
  cur[w] = b;
  pick[item * (W + 1) + w] = (int8_t)jb;
}

__global__ __launch_bounds__(kMckpThreads) void mckp_copy_kernel(const double *__restrict__ src,
                                                                 double *__restrict__ dst,
                                                                 int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * kMckpThreads + threadIdx.x;
  if (i < n) dst[i] = src[i];
}

// One lane: the budget search and the read-back of the selection.
__global__ void mckp_search_kernel(const int64_t *__restrict__ sizes, int64_t L, int nb,
                                   int64_t W, double tau, const double *__restrict__ best,
                                   const int8_t *__restrict__ pick, int32_t *__restrict__ choice,
                                   int64_t *__restrict__ result, double *__restrict__ cost) {
  if (blockIdx.x != 0 || threadIdx.x != 0) return;
  auto meets = [&](int64_t w) { return isfinite(best[w]) && best[w] <= tau; };
  int64_t status, budget;
  if (!meets(W)) {
    status = isinf(best[W]) ? 2 : 1;
    budget = W;
  } else {
    int64_t lo = 0, hi = W;   // budget hi meets the target
    while (lo < hi) {
      const int64_t mid = lo + (hi - lo) / 2;
      if (meets(mid)) hi = mid;
      else lo = mid + 1;
    }
    status = 0;
    budget = lo;
  }
  int64_t total = 0;
  if (status == 2) {
    for (int64_t l = 0; l < L; ++l) choice[l] = -1;
  } else {
    int64_t w = budget;
    for (int64_t l = L - 1; l >= 0; --l) {
      const int j = pick[l * (W + 1) + w];
      choice[l] = j;
      w -= sizes[l * nb + j];
      total += sizes[l * nb + j];
    }
  }
  result[0] = status;
  result[1] = status == 0 ? budget : -1;
  result[2] = status == 2 ? -1 : total;
  *cost = status == 2 ? INFINITY : best[budget];
}

}  // namespace

size_t mckp_workspace(int64_t L, int64_t W) {
  const size_t rows = (size_t)2 * (W + 1) * sizeof(double);
  return (rows + (size_t)L * (W + 1) + 255) / 256 * 256;
}

hipError_t launch_mckp(const int64_t *sizes, const double *costs, int64_t L, int nb, int64_t W,
                       double tau, int32_t *choice, int64_t *result, double *cost, double *best,
                       void *ws, hipStream_t s) {
  double *row[2] = {static_cast<double *>(ws), static_cast<double *>(ws) + (W + 1)};
  int8_t *pick = reinterpret_cast<int8_t *>(row[1] + (W + 1));
  const unsigned blocks = (unsigned)((W + 1 + kMckpThreads - 1) / kMckpThreads);
  hipLaunchKernelGGL(mckp_zero_kernel, dim3(blocks), dim3(kMckpThreads), 0, s, row[0], W + 1);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  for (int64_t l = 0; l < L; ++l) {
    hipLaunchKernelGGL(mckp_item_kernel, dim3(blocks), dim3(kMckpThreads), 0, s, sizes, costs, nb,
                       l, W, row[l & 1], row[(l + 1) & 1], pick);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const double *fin = row[L & 1];
  hipLaunchKernelGGL(mckp_search_kernel, dim3(1), dim3(64), 0, s, sizes, L, nb, W, tau, fin, pick,
                     choice, result, cost);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (best) {
    hipLaunchKernelGGL(mckp_copy_kernel, dim3(blocks), dim3(kMckpThreads), 0, s, fin, best, W + 1);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace slq
