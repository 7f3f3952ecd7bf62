// Prefill-path weight-only dequantize matmul (m > 64) for gfx950.
//
// y[m][n] = sum_k x[m][k] * w_hat[n][k] with w_hat = (q - z) * s per 128-group
// (gist.science summary "Statistically-Lossless Quantization of Large Language
// Models", Methodology 3 and Inference Speedup; SLQ README, Usage 4).
//
// With thousands of activation rows the product is a dense contraction and the
// bound is the bf16 MFMA rate.  Each workgroup computes a 128x128 tile of y:
// per 64-wide k step it stages the activation tile and the dequantized weight
// tile (packed codes -> (q - z) * s in fp32 -> bf16) in LDS, then four
// wavefronts each run a 4x4 grid of 16x16x32 bf16 MFMAs with fp32
// accumulation.  The weight tile is dequantized once per workgroup and reused
// by every activation row of the tile.
#include "launch.h"
#include "slq_device.h"

namespace slq {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 128;          // m and n extent of a workgroup tile
constexpr int kStep = 64;           // k per LDS stage
constexpr int kPitch = kStep + 8;   // bf16 elements per LDS row (padding vs bank conflicts)

__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) {
  const __bf16 a = (__bf16)lo, b = (__bf16)hi;   // round to nearest even
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

template <int BITS>
__global__ __launch_bounds__(kThreads) void gemm_kernel(
    const uint16_t *__restrict__ x, const uint32_t *__restrict__ codes,
    const float *__restrict__ scales, const uint8_t *__restrict__ zeros, int M, int N, int K,
    float *__restrict__ y) {
  __shared__ __attribute__((aligned(16))) uint16_t As[kTile * kPitch];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[kTile * kPitch];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int wm = wave / 2, wn = wave % 2;
  const int col = lane & 15, kq = lane >> 4;
  const int m0 = blockIdx.y * kTile, n0 = blockIdx.x * kTile;
  const int G = K / kGroup;
  const int64_t wpr = (int64_t)K * BITS / 32;

  // Staging roles: thread t fills row t/2, half t%2 (32 k) of both tiles.
  const int sr = threadIdx.x >> 1, sh = threadIdx.x & 1;
  const int xm = min(m0 + sr, M - 1);
  const int wnr = min(n0 + sr, N - 1);
  const uint16_t *xsrc = x + (int64_t)xm * K + 32 * sh;
  const uint32_t *csrc = codes + (int64_t)wnr * wpr + sh * BITS;
  const float *ssrc = scales + (int64_t)wnr * G;
  const uint8_t *zsrc = zeros + (int64_t)wnr * G;
  constexpr uint32_t mask = (1u << BITS) - 1u;

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < K; k0 += kStep) {
    // activations: 64 bytes per thread
    {
      const u32x4_t *px = reinterpret_cast<const u32x4_t *>(xsrc + k0);
      u32x4_t *dst = reinterpret_cast<u32x4_t *>(As + sr * kPitch + 32 * sh);
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[i] = px[i];
    }
    // weights: one 32-code chunk per thread, dequantized to bf16
    {
      const uint32_t *pc = csrc + (int64_t)(k0 / 32) * BITS;
      uint32_t w[BITS];
#pragma unroll
      for (int i = 0; i < BITS; ++i) w[i] = pc[i];
      const int g = k0 / kGroup;
      const float s = ssrc[g];
      const int z = zsrc[g];
      uint32_t out[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        uint32_t qv[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int bit = (2 * j + e) * BITS, wi = bit / 32, o = bit % 32;
          uint32_t v = w[wi] >> o;
          if (o + BITS > 32) v |= w[wi + 1] << (32 - o);
          qv[e] = v & mask;
        }
        out[j] = bf16_pair((float)((int)qv[0] - z) * s, (float)((int)qv[1] - z) * s);
      }
      u32x4_t *dst = reinterpret_cast<u32x4_t *>(Bs + sr * kPitch + 32 * sh);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        dst[i] = u32x4_t{out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]};
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < kStep / 32; ++ks) {
      u32x4_t a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = *reinterpret_cast<const u32x4_t *>(As + (64 * wm + 16 * i + col) * kPitch + 32 * ks + 8 * kq);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[j] = *reinterpret_cast<const u32x4_t *>(Bs + (64 * wn + 16 * j + col) * kPitch + 32 * ks + 8 * kq);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + 64 * wn + 16 * j + col;
      if (n >= N) continue;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = m0 + 64 * wm + 16 * i + 4 * kq + v;
        if (m < M) y[(int64_t)m * N + n] = acc[i][j][v];
      }
    }
}

template <int BITS>
hipError_t gemm_bits(const uint16_t *x, const uint32_t *codes, const float *scales,
                     const uint8_t *zeros, int64_t m, int64_t n, int64_t k, float *y,
                     hipStream_t st) {
  const dim3 grid((unsigned)((n + kTile - 1) / kTile), (unsigned)((m + kTile - 1) / kTile));
  hipLaunchKernelGGL((gemm_kernel<BITS>), grid, dim3(kThreads), 0, st, x, codes, scales, zeros,
                     (int)m, (int)n, (int)k, y);
  return hipGetLastError();
}

}  // namespace

size_t gemm_workspace(int64_t, int64_t, int64_t, int) { return 0; }

hipError_t launch_gemm(const uint16_t *x, const uint32_t *codes, const float *scales,
                       const uint8_t *zeros, int64_t m, int64_t n, int64_t k, int bits, float *y,
                       void *, hipStream_t s) {
  switch (bits) {
    case 2: return gemm_bits<2>(x, codes, scales, zeros, m, n, k, y, s);
    case 3: return gemm_bits<3>(x, codes, scales, zeros, m, n, k, y, s);
    case 4: return gemm_bits<4>(x, codes, scales, zeros, m, n, k, y, s);
    case 5: return gemm_bits<5>(x, codes, scales, zeros, m, n, k, y, s);
    case 6: return gemm_bits<6>(x, codes, scales, zeros, m, n, k, y, s);
    case 7: return gemm_bits<7>(x, codes, scales, zeros, m, n, k, y, s);
    case 8: return gemm_bits<8>(x, codes, scales, zeros, m, n, k, y, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace slq
