// Group quantization with dense bit-packing, reconstruction, and the
// quantization-noise sums behind the gamma-squared law, for gfx950.
//
// Method (gist.science summary "Statistically-Lossless Quantization of Large
// Language Models", Methodology 3: asymmetric integer group quantization with
// group size 128; Methodology 1: the symmetric grid as the comparison and the
// centering inefficiency gamma = 2M/R; SLQ README, Pipeline: bit-widths 2..8;
// Usage 4: weights packed to their per-layer bit-width).
//
// Work decomposition: one lane owns one 32-code chunk of a row (the unit the
// packed layout is built from: 32 codes fill exactly `bits` 32-bit words), so
// a 128-group is four consecutive lanes of one wavefront.  The group's min/max
// is two cross-lane steps; codes are packed in registers and stored as `bits`
// consecutive words per lane, contiguous across lanes.
//
// Every fp32 step (subtract, divide, round-half-even) is a single IEEE
// correctly rounded operation with no contraction, so codes, scales and zero
// points are bit-identical to any other IEEE implementation of the same steps.
#include "launch.h"
#include "slq_device.h"

namespace slq {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float clamp_code(float v, float maxq) {
  v = (v < 0.0f) ? 0.0f : v;
  return (v > maxq) ? maxq : v;
}

template <int BITS>
__device__ __forceinline__ void pack32(const uint32_t (&q)[32], uint32_t (&out)[BITS]) {
#pragma unroll
  for (int i = 0; i < BITS; ++i) out[i] = 0u;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const int bit = j * BITS, w = bit / 32, o = bit % 32;
    out[w] |= q[j] << o;
    if (o + BITS > 32) out[w + 1] |= q[j] >> (32 - o);
  }
}

template <int BITS>
__device__ __forceinline__ void unpack32(const uint32_t (&in)[BITS], uint32_t (&q)[32]) {
  constexpr uint32_t mask = (1u << BITS) - 1u;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const int bit = j * BITS, w = bit / 32, o = bit % 32;
    uint32_t v = in[w] >> o;
    if (o + BITS > 32) v |= in[w + 1] << (32 - o);
    q[j] = v & mask;
  }
}

template <int BITS>
__device__ __forceinline__ void load_words(const uint32_t *__restrict__ p, uint32_t (&w)[BITS]) {
#pragma unroll
  for (int i = 0; i < BITS; ++i) w[i] = p[i];
}

// CM: compact metadata (see MetaRd): the fp32 scale is rounded up to binary16
// and the zero point and codes are computed with the rounded scale.
template <int BITS, bool SYM, bool CM>
__global__ __launch_bounds__(kThreads) void quantize_pack_kernel(
    const float *__restrict__ W, int64_t chunks, uint32_t *__restrict__ codes,
    void *__restrict__ scales, uint8_t *__restrict__ zeros) {
  constexpr int maxq_i = (1 << BITS) - 1;
  const float maxq = (float)maxq_i;
  const int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  // chunks is a multiple of 4 and groups are 4 aligned lanes, so a group's
  // lanes are either all in range or all out of range.
  const int64_t cc = c < chunks ? c : chunks - 1;

  float w[32];
  const float4 *src = reinterpret_cast<const float4 *>(W + cc * 32);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float4 v = src[i];
    w[4 * i + 0] = v.x;
    w[4 * i + 1] = v.y;
    w[4 * i + 2] = v.z;
    w[4 * i + 3] = v.w;
  }

  float s, zf;
  if constexpr (!SYM) {
    float lo = 0.0f, hi = 0.0f;   // the range always contains 0
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      lo = (w[i] < lo) ? w[i] : lo;
      hi = (w[i] > hi) ? w[i] : hi;
    }
#pragma unroll
    for (int o = 1; o <= 2; o <<= 1) {
      float l2 = __shfl_xor(lo, o, kWave), h2 = __shfl_xor(hi, o, kWave);
      lo = (l2 < lo) ? l2 : lo;
      hi = (h2 > hi) ? h2 : hi;
    }
    const float range = hi - lo;
    s = range / maxq;
    if (s == 0.0f) {   // all-zero group (or a range that underflows)
      s = 1.0f;
      zf = 0.0f;
    } else {
      if constexpr (CM) s = f16_bits_to_f32(f16_bits_round_up(s));
      zf = clamp_code(rintf((-lo) / s), maxq);
    }
  } else {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const float a = fabsf(w[i]);
      m = (a > m) ? a : m;
    }
#pragma unroll
    for (int o = 1; o <= 2; o <<= 1) {
      const float m2 = __shfl_xor(m, o, kWave);
      m = (m2 > m) ? m2 : m;
    }
    const float two_m = 2.0f * m;
    s = two_m / maxq;
    if (s == 0.0f) s = 1.0f;
    if constexpr (CM) s = f16_bits_to_f32(f16_bits_round_up(s));
    zf = (float)(1 << (BITS - 1));
  }

  uint32_t q[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const float t = rintf(w[i] / s);
    q[i] = (uint32_t)(int)clamp_code(t + zf, maxq);
  }
  uint32_t packed[BITS];
  pack32<BITS>(q, packed);

  // nibble zero points: the first lane of an even group also takes the odd
  // group's zero point (4 lanes on; 0 past the last group)
  uint32_t zodd = 0;
  if constexpr (CM && BITS <= 4) {
    zodd = (uint32_t)(int)__shfl_down(zf, 4, kWave);
    if (c + 4 >= chunks) zodd = 0;
  }
  if (c < chunks) {
    uint32_t *dst = codes + c * BITS;
#pragma unroll
    for (int i = 0; i < BITS; ++i) dst[i] = packed[i];
    if ((c & 3) == 0) {
      if constexpr (CM) {
        // s is already a binary16 value: rounding it up returns its own bits
        static_cast<uint16_t *>(scales)[c >> 2] = (uint16_t)f16_bits_round_up(s);
        if constexpr (BITS <= 4) {
          if ((c & 7) == 0) zeros[c >> 3] = (uint8_t)((uint32_t)(int)zf | (zodd << 4));
        } else {
          zeros[c >> 2] = (uint8_t)(int)zf;
        }
      } else {
        static_cast<float *>(scales)[c >> 2] = s;
        zeros[c >> 2] = (uint8_t)(int)zf;
      }
    }
  }
}

template <int BITS, bool CM>
__global__ __launch_bounds__(kThreads) void dequantize_kernel(
    const uint32_t *__restrict__ codes, const void *__restrict__ scales,
    const uint8_t *__restrict__ zeros, int64_t chunks, float *__restrict__ out) {
  const MetaRd<BITS, CM> meta{scales, zeros};
  const int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (c >= chunks) return;
  uint32_t words[BITS], q[32];
  load_words<BITS>(codes + c * BITS, words);
  unpack32<BITS>(words, q);
  const float s = meta.scale(c >> 2);
  const int z = (int)meta.zero(c >> 2);
  float4 *dst = reinterpret_cast<float4 *>(out + c * 32);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float4 v;
    v.x = (float)((int)q[4 * i + 0] - z) * s;
    v.y = (float)((int)q[4 * i + 1] - z) * s;
    v.z = (float)((int)q[4 * i + 2] - z) * s;
    v.w = (float)((int)q[4 * i + 3] - z) * s;
    dst[i] = v;
  }
}

__device__ __forceinline__ double block_sum_f64(double v, double *lds) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  const int wave = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) lds[wave] = v;
  __syncthreads();
  double t = 0.0;
  if (threadIdx.x == 0)
    for (int i = 0; i < kThreads / kWave; ++i) t += lds[i];
  return t;
}

// Per block: sum (w - w_hat)^2 over its chunks and sum s^2 over its groups.
template <int BITS, bool CM>
__global__ __launch_bounds__(kThreads) void quant_error_kernel(
    const float *__restrict__ W, const uint32_t *__restrict__ codes,
    const void *__restrict__ scales, const uint8_t *__restrict__ zeros, int64_t chunks,
    double *__restrict__ partial) {
  __shared__ double lds[kThreads / kWave];
  const MetaRd<BITS, CM> meta{scales, zeros};
  const int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  double sse = 0.0, s2 = 0.0;
  if (c < chunks) {
    uint32_t words[BITS], q[32];
    load_words<BITS>(codes + c * BITS, words);
    unpack32<BITS>(words, q);
    const float s = meta.scale(c >> 2);
    const int z = (int)meta.zero(c >> 2);
    const float4 *src = reinterpret_cast<const float4 *>(W + c * 32);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float4 v = src[i];
      const float wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float wh = (float)((int)q[4 * i + j] - z) * s;
        const double d = (double)wv[j] - (double)wh;
        sse += d * d;
      }
    }
    if ((c & 3) == 0) s2 = (double)s * (double)s;
  }
  const double a = block_sum_f64(sse, lds);
  const double b = block_sum_f64(s2, lds);
  if (threadIdx.x == 0) {
    partial[2 * blockIdx.x + 0] = a;
    partial[2 * blockIdx.x + 1] = b;
  }
}

// Fixed-order sum of the per-block partials: thread t adds blocks t, t+256, ...
__global__ __launch_bounds__(kThreads) void sum_pairs_kernel(const double *__restrict__ partial,
                                                             int64_t nblocks,
                                                             double *__restrict__ out) {
  __shared__ double lds[kThreads / kWave];
  double a = 0.0, b = 0.0;
  for (int64_t i = threadIdx.x; i < nblocks; i += kThreads) {
    a += partial[2 * i + 0];
    b += partial[2 * i + 1];
  }
  const double ta = block_sum_f64(a, lds);
  const double tb = block_sum_f64(b, lds);
  if (threadIdx.x == 0) {
    out[0] = ta;
    out[1] = tb;
  }
}

template <int BITS>
hipError_t quantize_bits(const float *W, int64_t chunks, bool sym, bool cm, uint32_t *codes,
                         void *scales, uint8_t *zeros, hipStream_t st) {
  const dim3 grid((unsigned)((chunks + kThreads - 1) / kThreads));
#define SLQ_Q(SYM_, CM_)                                                                       \
  hipLaunchKernelGGL((quantize_pack_kernel<BITS, SYM_, CM_>), grid, dim3(kThreads), 0, st, W, \
                     chunks, codes, scales, zeros)
  if (sym) {
    if (cm) SLQ_Q(true, true);
    else SLQ_Q(true, false);
  } else {
    if (cm) SLQ_Q(false, true);
    else SLQ_Q(false, false);
  }
#undef SLQ_Q
  return hipGetLastError();
}

template <int BITS>
hipError_t dequantize_bits(const uint32_t *codes, const void *scales, const uint8_t *zeros,
                           bool cm, int64_t chunks, float *out, hipStream_t st) {
  const dim3 grid((unsigned)((chunks + kThreads - 1) / kThreads));
  if (cm)
    hipLaunchKernelGGL((dequantize_kernel<BITS, true>), grid, dim3(kThreads), 0, st, codes,
                       scales, zeros, chunks, out);
  else
    hipLaunchKernelGGL((dequantize_kernel<BITS, false>), grid, dim3(kThreads), 0, st, codes,
                       scales, zeros, chunks, out);
  return hipGetLastError();
}

template <int BITS>
hipError_t quant_error_bits(const float *W, const uint32_t *codes, const void *scales,
                            const uint8_t *zeros, bool cm, int64_t chunks, double *out,
                            double *partial, hipStream_t st) {
  const int64_t nblocks = (chunks + kThreads - 1) / kThreads;
  if (nblocks > 0) {
    if (cm)
      hipLaunchKernelGGL((quant_error_kernel<BITS, true>), dim3((unsigned)nblocks), dim3(kThreads),
                         0, st, W, codes, scales, zeros, chunks, partial);
    else
      hipLaunchKernelGGL((quant_error_kernel<BITS, false>), dim3((unsigned)nblocks),
                         dim3(kThreads), 0, st, W, codes, scales, zeros, chunks, partial);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(sum_pairs_kernel, dim3(1), dim3(kThreads), 0, st, partial, nblocks, out);
  return hipGetLastError();
}

}  // namespace

#define SLQ_DISPATCH_BITS(bits, F, ...)        \
  switch (bits) {                              \
    case 2: return F<2>(__VA_ARGS__);          \
    case 3: return F<3>(__VA_ARGS__);          \
    case 4: return F<4>(__VA_ARGS__);          \
    case 5: return F<5>(__VA_ARGS__);          \
    case 6: return F<6>(__VA_ARGS__);          \
    case 7: return F<7>(__VA_ARGS__);          \
    case 8: return F<8>(__VA_ARGS__);          \
    default: return hipErrorInvalidValue;      \
  }

hipError_t launch_quantize_pack(const float *W, int64_t n, int64_t k, int bits, bool symmetric,
                                bool compact, uint32_t *codes, void *scales, uint8_t *zeros,
                                hipStream_t s) {
  const int64_t chunks = n * (k / 32);
  if (chunks == 0) return hipSuccess;
  SLQ_DISPATCH_BITS(bits, quantize_bits, W, chunks, symmetric, compact, codes, scales, zeros, s);
}

hipError_t launch_dequantize(const uint32_t *codes, const void *scales, const uint8_t *zeros,
                             bool compact, int64_t n, int64_t k, int bits, float *out,
                             hipStream_t s) {
  const int64_t chunks = n * (k / 32);
  if (chunks == 0) return hipSuccess;
  SLQ_DISPATCH_BITS(bits, dequantize_bits, codes, scales, zeros, compact, chunks, out, s);
}

size_t quant_error_workspace(int64_t n, int64_t k) {
  const int64_t chunks = n * (k / 32);
  return (size_t)((chunks + kThreads - 1) / kThreads) * 2 * sizeof(double);
}

hipError_t launch_quant_error(const float *W, const uint32_t *codes, const void *scales,
                              const uint8_t *zeros, bool compact, int64_t n, int64_t k, int bits,
                              double *out, void *ws, hipStream_t s) {
  const int64_t chunks = n * (k / 32);
  SLQ_DISPATCH_BITS(bits, quant_error_bits, W, codes, scales, zeros, compact, chunks, out,
                    static_cast<double *>(ws), s);
}

}  // namespace slq
