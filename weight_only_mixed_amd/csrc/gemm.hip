// Prefill-path weight-only dequantize matmul (m > 64) for gfx950.
//
// y[m][n] = sum_k x[m][k] * w_hat[n][k] with w_hat = (q - z) * s per 128-group
// (gist.science summary "Statistically-Lossless Quantization of Large Language
// Models", Methodology 3 and Inference Speedup; SLQ README, Usage 4).
//
// With thousands of activation rows the product is a dense contraction bound
// by the bf16 MFMA rate, so the design keeps the matrix cores fed and moves
// the dequantization off the LDS path:
//  * A workgroup computes a kBM (m) x 256 (n) tile of y with four wavefronts;
//    wavefront w owns columns [64w, 64w + 64) and all kBM rows, as a kMT x 2
//    grid of 32x32x16 bf16 MFMAs with fp32 accumulators.
//  * Activations: the kBM x 64 tile of each k step is staged in LDS (double
//    buffered) and read as the A operands; its global loads are issued two
//    steps ahead.
//  * Weights never pass through LDS: each lane loads the 32-code chunk of its
//    column for its half of the k step straight into registers (one chunk per
//    32-column MFMA tile, prefetched two steps ahead) and dequantizes it into the
//    B operands: w_hat = fl32((q - z) * s) with one fma per code (see Deq),
//    rounded to bf16.
//    Every weight code is dequantized by exactly one lane.  The MFMA k slots
//    are assigned so that a lane's 8 slots of the 4 MFMA steps of a k step
//    are its chunk's 32 consecutive codes; the A operands read the matching
//    activations from LDS.
//
// Two kernels share this scheme.  gemm_wide_kernel (256 x 256 tiles, one
// wavefront per SIMD, each dequantized operand feeding 8 MFMAs) serves grids
// that fill the chip, and smaller grids with m >= 1024 by splitting k over the
// grid's z dimension (partial tiles summed in order by a second kernel);
// gemm_kernel (128 x 256 tiles, two wavefronts per SIMD) serves the rest.
#include <algorithm>

#include "launch.h"
#include "slq_device.h"

namespace slq {
namespace {

constexpr int kThreads = 256;
#ifndef SLQ_GEMM_MTILES
#define SLQ_GEMM_MTILES 4
#endif
#ifndef SLQ_GEMM_NTILES
#define SLQ_GEMM_NTILES 2
#endif
#ifndef SLQ_GEMM_WAVES_M
#define SLQ_GEMM_WAVES_M 1
#endif
constexpr int kMT = SLQ_GEMM_MTILES;    // 32-row MFMA tiles per wavefront
constexpr int kNTW = SLQ_GEMM_NTILES;   // 32-column MFMA tiles per wavefront
constexpr int kWM = SLQ_GEMM_WAVES_M;   // wavefronts along m (the rest along n)
constexpr int kWN = 4 / kWM;
constexpr int kBM = 32 * kMT * kWM;     // m extent of a workgroup tile
constexpr int kBN = 32 * kNTW * kWN;    // n extent of a workgroup tile
constexpr int kBK = 64;                 // k per step
constexpr int kPitch = kBK + 8;         // bf16 elements per LDS row (padding vs bank conflicts)
constexpr size_t kLdsBytes = (size_t)2 * kBM * kPitch * 2;

typedef float f32x16_t __attribute__((ext_vector_type(16)));

// 32x32x16 bf16 MFMA: D[32x32] += A[32x16] * B[16x32], fp32 accumulate.
// Lane l supplies A row (l % 32) and B column (l % 32), k slots 8*(l/32)+t;
// it receives D[8*(i/4) + 4*(l/32) + i%4][l % 32] in element i.
__device__ __forceinline__ f32x16_t mfma32(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two fp32 values -> one packed bf16 pair, round to nearest even (a single
// v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

template <int BITS>
struct Chunk {
  uint32_t w[BITS];
};

template <int BITS>
__device__ __forceinline__ Chunk<BITS> load_chunk(const uint32_t *__restrict__ p) {
  Chunk<BITS> c;
  if constexpr (BITS % 4 == 0) {
#pragma unroll
    for (int i = 0; i < BITS / 4; ++i) {
      const u32x4_t v = reinterpret_cast<const u32x4_t *>(p)[i];
      c.w[4 * i + 0] = v[0];
      c.w[4 * i + 1] = v[1];
      c.w[4 * i + 2] = v[2];
      c.w[4 * i + 3] = v[3];
    }
  } else if constexpr (BITS % 2 == 0) {
#pragma unroll
    for (int i = 0; i < BITS / 2; ++i) {
      const u32x2_t v = reinterpret_cast<const u32x2_t *>(p)[i];
      c.w[2 * i + 0] = v[0];
      c.w[2 * i + 1] = v[1];
    }
  } else {
#pragma unroll
    for (int i = 0; i < BITS; ++i) c.w[i] = p[i];
  }
  return c;
}

// w_hat = fl32((q - z) * s) exactly as the definition rounds it, one fma per
// code: for widths up to 7, u = q - z + 128 is a positive integer below 256
// (so it is formed with integer adds, byte-parallel where codes sit in bytes,
// and converted exactly), and fma(u, s, -128 s) computes (q - z) s with a
// single rounding because -128 s is exact.  8-bit codes subtract z in fp32
// (exact) and multiply.
struct Deq {
  float s;       // scale
  float c0;      // -128 * s
  float zf;      // z (8-bit path)
  uint32_t zo;   // 128 - z in every byte
};

__device__ __forceinline__ Deq make_deq(float s, uint32_t z) {
  Deq d;
  d.s = s;
  d.c0 = -128.f * s;
  d.zf = (float)z;
  d.zo = (128u - z) * 0x01010101u;
  return d;
}

// Codes j of a chunk, offset by 128 - z, as exact floats (BITS <= 7).
template <int BITS>
__device__ __forceinline__ float code_u(const Chunk<BITS> &c, int j, uint32_t zo) {
  const int bit = j * BITS, wi = bit / 32, o = bit % 32;
  uint32_t v;
  if (o + BITS <= 32) v = (c.w[wi] >> o) & ((1u << BITS) - 1u);
  else v = alignbit(c.w[wi + 1], c.w[wi], o) & ((1u << BITS) - 1u);
  return (float)(v + (zo & 0xFFu));
}

// B operand of MFMA k-slice ks (codes 8ks..8ks+7 of the lane's chunk) for
// one 32-column tile, dequantized and rounded to bf16.
template <int BITS>
__device__ __forceinline__ u32x4_t dequant_slice(const Chunk<BITS> &c, const Deq &d, int ks) {
  uint32_t p[4];
  if constexpr (BITS == 4) {
    // codes in bytes: lo holds codes 0,2,4,6 of word ks, hi codes 1,3,5,7
    const uint32_t lo = (c.w[ks] & 0x0F0F0F0Fu) + d.zo, hi = ((c.w[ks] >> 4) & 0x0F0F0F0Fu) + d.zo;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float u0 = (float)((lo >> (8 * e)) & 0xFFu), u1 = (float)((hi >> (8 * e)) & 0xFFu);
      p[e] = bf16_pair(fmaf(u0, d.s, d.c0), fmaf(u1, d.s, d.c0));
    }
  } else if constexpr (BITS == 2) {
    // word ks/2 holds codes 16(ks/2)..+15; bytes of (word >> 2j) & 0x03.. hold codes 4b+j
    const uint32_t w = c.w[ks / 2];
    uint32_t by[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) by[j] = ((w >> (2 * j)) & 0x03030303u) + d.zo;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int k0 = 8 * (ks % 2) + 2 * e, k1 = k0 + 1;   // codes of the word
      const float u0 = (float)((by[k0 % 4] >> (8 * (k0 / 4))) & 0xFFu);
      const float u1 = (float)((by[k1 % 4] >> (8 * (k1 / 4))) & 0xFFu);
      p[e] = bf16_pair(fmaf(u0, d.s, d.c0), fmaf(u1, d.s, d.c0));
    }
  } else if constexpr (BITS == 8) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t w = c.w[2 * ks + e / 2];
      const float q0 = (float)((w >> (16 * (e % 2))) & 0xFFu);
      const float q1 = (float)((w >> (16 * (e % 2) + 8)) & 0xFFu);
      p[e] = bf16_pair((q0 - d.zf) * d.s, (q1 - d.zf) * d.s);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      p[e] = bf16_pair(fmaf(code_u<BITS>(c, 8 * ks + 2 * e, d.zo), d.s, d.c0),
                       fmaf(code_u<BITS>(c, 8 * ks + 2 * e + 1, d.zo), d.s, d.c0));
  }
  return u32x4_t{p[0], p[1], p[2], p[3]};
}

template <int BITS, bool CM>
__global__ __launch_bounds__(kThreads, kMT * kNTW > 8 ? 1 : 2) void gemm_kernel(
    const uint16_t *__restrict__ x, const uint32_t *__restrict__ codes,
    const void *__restrict__ scales, const uint8_t *__restrict__ zeros, int M, int N, int K,
    float *__restrict__ y) {
  const MetaRd<BITS, CM> md{scales, zeros};
  extern __shared__ __attribute__((aligned(16))) uint16_t lds_x[];
  uint16_t *As[2] = {lds_x, lds_x + kBM * kPitch};

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int wm = wave / kWN, wn = wave % kWN;
  const int c32 = lane & 31, h = lane >> 5;
  const int m0 = blockIdx.y * kBM, n0 = blockIdx.x * kBN + 32 * kNTW * wn;
  const int am = 32 * kMT * wm;   // first LDS activation row of this wave
  const int G = K / kGroup;
  const int64_t wpr = (int64_t)K * BITS / 32;
  const int steps = K / kBK;

  // activation staging: thread t copies rows t/2 + 128r, k half t%2 (64 bytes each)
  constexpr int XR = kBM / 128;
  const int sr = threadIdx.x >> 1, sh = threadIdx.x & 1;
  const u32x4_t *xsrc[XR];
#pragma unroll
  for (int r = 0; r < XR; ++r)
    xsrc[r] = reinterpret_cast<const u32x4_t *>(x + (int64_t)min(m0 + sr + 128 * r, M - 1) * K + 32 * sh);
  auto load_x = [&](int st, u32x4_t (&v)[XR][4]) {
#pragma unroll
    for (int r = 0; r < XR; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i) v[r][i] = xsrc[r][st * (kBK / 8) + i];
  };
  auto store_x = [&](int buf, const u32x4_t (&v)[XR][4]) {
#pragma unroll
    for (int r = 0; r < XR; ++r) {
      u32x4_t *dst = reinterpret_cast<u32x4_t *>(&As[buf][(sr + 128 * r) * kPitch + 32 * sh]);
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[i] = v[r][i];
    }
  };

  // weights: column n = n0 + 32t + c32 (rows past N are read, never stored);
  // the lane's chunk of step st is chunk 2*st + h of the row
  const uint32_t *crow[kNTW];
  int64_t mrow[kNTW];   // flat group index of the row's first group
#pragma unroll
  for (int t = 0; t < kNTW; ++t) {
    const int n = min(n0 + 32 * t + c32, N - 1);
    crow[t] = codes + (int64_t)n * wpr + h * BITS;
    mrow[t] = (int64_t)n * G;
  }
  // chunks, scale and zero point of step st (a step is half a 128-group)
  auto load_w = [&](int st, Chunk<BITS> (&c)[kNTW], float (&sv)[kNTW], uint32_t (&zv)[kNTW]) {
    const int g = (st * kBK) / kGroup;
#pragma unroll
    for (int t = 0; t < kNTW; ++t) {
      c[t] = load_chunk<BITS>(crow[t] + (int64_t)st * 2 * BITS);
      sv[t] = md.scale(mrow[t] + g);
      zv[t] = md.zero(mrow[t] + g);
    }
  };

  f32x16_t acc[kMT][kNTW];
#pragma unroll
  for (int i = 0; i < kMT; ++i)
#pragma unroll
    for (int t = 0; t < kNTW; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][t][e] = 0.f;

  // Prefetch ahead: a step's activation tile is requested two steps before it
  // is needed and its weight chunks one and a half steps before, which covers
  // an HBM round trip under load.  Two register sets of each alternate between even
  // and odd steps (no copies: copying a register with a load in flight would
  // wait for it); loads complete in issue order, so waiting for x(st+1) at
  // the end of step st does not wait for the step-st requests.
  u32x4_t xA[XR][4], xB[XR][4];
  Chunk<BITS> wA[kNTW], wB[kNTW];
  float sA[kNTW], sB[kNTW];
  uint32_t zA[kNTW], zB[kNTW];
  load_x(0, xA);
  store_x(0, xA);
  load_w(0, wA, sA, zA);
  load_w(1, wB, sB, zB);   // steps = 2 * groups >= 2
  load_x(1, xB);
  __syncthreads();

  // step st: issue x(st+2) into xi, run the MFMAs on w (= w(st)) dequantized
  // slice by slice, refill that slot with w(st+2), store xs (= x(st+1)) to the
  // other buffer
  auto step = [&](int st, u32x4_t (&xi)[XR][4], const u32x4_t (&xs)[XR][4], Chunk<BITS> (&w)[kNTW],
                  float (&sw)[kNTW], uint32_t (&zw)[kNTW]) {
    const int buf = st & 1;
    const int n2 = min(st + 2, steps - 1);   // past the end: reload the last step (discarded)
    load_x(n2, xi);
    __builtin_amdgcn_sched_barrier(0);   // keep the prefetch ahead of the MFMAs
    Deq d[kNTW];
#pragma unroll
    for (int t = 0; t < kNTW; ++t) d[t] = make_deq(sw[t], zw[t]);
    // k slots 8h+t of MFMA slice ks <-> k = 32h + 8ks + t within the step; the
    // A operands of slice ks+1 are read from LDS before slice ks's MFMAs
    auto read_a = [&](int ks, u32x4_t (&a)[kMT]) {
#pragma unroll
      for (int i = 0; i < kMT; ++i)
        a[i] = *reinterpret_cast<const u32x4_t *>(&As[buf][(am + 32 * i + c32) * kPitch + 32 * h + 8 * ks]);
    };
    u32x4_t a0[kMT], a1[kMT];
    read_a(0, a0);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4_t(&a)[kMT] = (ks & 1) ? a1 : a0;
      u32x4_t(&an)[kMT] = (ks & 1) ? a0 : a1;
      if (ks + 1 < 4) read_a(ks + 1, an);
      u32x4_t b[kNTW];
#pragma unroll
      for (int t = 0; t < kNTW; ++t) b[t] = dequant_slice<BITS>(w[t], d[t], ks);
#pragma unroll
      for (int i = 0; i < kMT; ++i)
#pragma unroll
        for (int t = 0; t < kNTW; ++t) acc[i][t] = mfma32(a[i], b[t], acc[i][t]);
    }
    load_w(n2, w, sw, zw);   // the slot is free once its last slice is dequantized
    if (st + 1 < steps) store_x(buf ^ 1, xs);
    __syncthreads();
  };
  for (int st = 0; st < steps; st += 2) {
    step(st, xA, xB, wA, sA, zA);
    step(st + 1, xB, xA, wB, sB, zB);
  }

#pragma unroll
  for (int t = 0; t < kNTW; ++t) {
    const int n = n0 + 32 * t + c32;
    if (n >= N) continue;
#pragma unroll
    for (int i = 0; i < kMT; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + am + 32 * i + 8 * (e / 4) + 4 * h + (e % 4);
        if (m < M) y[(int64_t)m * N + n] = acc[i][t][e];
      }
  }
}

// ---- Wide tiles: 256 (m) x 256 (n), one wavefront per SIMD ----
//
// Wavefront w owns columns [64w, 64w + 64) and all 256 rows (8 x 2 MFMA
// tiles, 256 fp32 accumulators in the accumulation registers), so every
// dequantized B operand feeds eight MFMAs: half the dequantization work per
// MFMA of the 128-row tiles, which matters because the unpack, the fma and
// the bf16 conversion run on the VALU at ~3 instructions per code.
// With one wavefront per SIMD nothing else hides latency, so the operands of
// slice s+1 (A from LDS, B dequantized from registers) are produced while the
// 16 MFMAs of slice s run, including across step boundaries: the activation
// tile goes through three LDS buffers (written two steps ahead), so the A
// operands of the next step's first slice can be read before the step's
// closing barrier.
constexpr int kWideMT = 8;                  // 32-row MFMA tiles per wavefront
constexpr int kWideBM = 32 * kWideMT;       // 256
constexpr int kWideBN = 256;
constexpr int kWideBuf = kWideBM * kPitch;  // bf16 elements per LDS buffer
constexpr size_t kWideLdsBytes = (size_t)3 * kWideBuf * 2;
// Split-k partial tiles start past the workspace's first 64 KiB, which hold
// the decode path's split-k tickets (kept zero between calls).
constexpr size_t kGemmPartOffset = 65536;
constexpr int64_t kMaxGridY = 65535;   // workgroups along a grid's y dimension

// VALU instructions to place after each MFMA (the dequantization of one
// 8-code B slice per 32-column tile, spread over the 16 MFMAs of a slice).
// Measured on the 70B q/o and gate shapes at M = 4096: 3 and 5 run 3-6%
// faster than 4 and 6, and than 2/4, 3/4, 3/6, 4/5 or 5/7 (the rest of a
// slice's dequantization trails its MFMAs).
#ifndef SLQ_GEMM_WIDE_VPM_POW2
#define SLQ_GEMM_WIDE_VPM_POW2 3   // widths 2, 4 and 8
#endif
#ifndef SLQ_GEMM_WIDE_VPM_ODD
#define SLQ_GEMM_WIDE_VPM_ODD 5    // widths 3, 5, 6 and 7
#endif
template <int BITS>
constexpr int wide_valu_per_mfma() {
  return (BITS == 2 || BITS == 4 || BITS == 8) ? SLQ_GEMM_WIDE_VPM_POW2 : SLQ_GEMM_WIDE_VPM_ODD;
}

template <int BITS, bool CM>
__global__ __launch_bounds__(kThreads, 1) void gemm_wide_kernel(
    const uint16_t *__restrict__ x, const uint32_t *__restrict__ codes,
    const void *__restrict__ scales, const uint8_t *__restrict__ zeros, int M, int N, int K,
    int ksteps, float *__restrict__ y, float *__restrict__ part) {
  const MetaRd<BITS, CM> md{scales, zeros};
  extern __shared__ __attribute__((aligned(16))) uint16_t lds_x[];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int c32 = lane & 31, h = lane >> 5;
  const int m0 = blockIdx.y * kWideBM, n0 = blockIdx.x * kWideBN + 64 * wave;
  const int G = K / kGroup;
  const int64_t wpr = (int64_t)K * BITS / 32;
  // split k: this workgroup's k steps [st0, st0 + steps) (an even count >= 2);
  // with several splits the fp32 partial tile goes to part[blockIdx.z]
  const int st0 = blockIdx.z * ksteps;
  const int steps = min(ksteps, K / kBK - st0);
  float *__restrict__ out = part ? part + (int64_t)blockIdx.z * M * N : y;

  // activation staging: thread t copies rows t/2 and t/2 + 128, k half t%2
  const int sr = threadIdx.x >> 1, sh = threadIdx.x & 1;
  const u32x4_t *xsrc[2];
#pragma unroll
  for (int r = 0; r < 2; ++r)
    xsrc[r] = reinterpret_cast<const u32x4_t *>(x + (int64_t)min(m0 + sr + 128 * r, M - 1) * K +
                                                 (int64_t)st0 * kBK + 32 * sh);
  auto load_x = [&](int st, u32x4_t (&v)[2][4]) {
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i) v[r][i] = xsrc[r][st * (kBK / 8) + i];
  };
  auto store_x = [&](int b, const u32x4_t (&v)[2][4]) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      u32x4_t *dst = reinterpret_cast<u32x4_t *>(&lds_x[b * kWideBuf + (sr + 128 * r) * kPitch + 32 * sh]);
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[i] = v[r][i];
    }
  };

  // weights: as in gemm_kernel, column n0 + 32t + c32, chunk 2*(st0 + st) + h of the row
  const uint32_t *crow[2];
  int64_t mrow[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int n = min(n0 + 32 * t + c32, N - 1);
    crow[t] = codes + (int64_t)n * wpr + (int64_t)st0 * 2 * BITS + h * BITS;
    mrow[t] = (int64_t)n * G + st0 * kBK / kGroup;
  }
  auto load_w = [&](int st, Chunk<BITS> (&c)[2], float (&sv)[2], uint32_t (&zv)[2]) {
    const int g = (st * kBK) / kGroup;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      c[t] = load_chunk<BITS>(crow[t] + (int64_t)st * 2 * BITS);
      sv[t] = md.scale(mrow[t] + g);
      zv[t] = md.zero(mrow[t] + g);
    }
  };
  // A operands of slice ks from LDS buffer b
  auto read_a = [&](int b, int ks, u32x4_t (&a)[kWideMT]) {
#pragma unroll
    for (int i = 0; i < kWideMT; ++i)
      a[i] = *reinterpret_cast<const u32x4_t *>(&lds_x[b * kWideBuf + (32 * i + c32) * kPitch + 32 * h + 8 * ks]);
  };

  f32x16_t acc[kWideMT][2];
#pragma unroll
  for (int i = 0; i < kWideMT; ++i)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][t][e] = 0.f;

  // Prologue: x(0), x(1) into buffers 0 and 1; weights of steps 0 and 1;
  // the first slice's operands.
  u32x4_t xr[2][4];
  Chunk<BITS> wA[2], wB[2];
  float sA[2], sB[2];
  uint32_t zA[2], zB[2];
  load_x(0, xr);
  load_w(0, wA, sA, zA);
  load_w(1, wB, sB, zB);   // steps = 2 * groups >= 2
  store_x(0, xr);
  load_x(1, xr);
  store_x(1, xr);
  __syncthreads();
  u32x4_t a0[kWideMT], a1[kWideMT], b0[2], b1[2];
  read_a(0, 0, a0);
#pragma unroll
  for (int t = 0; t < 2; ++t) b0[t] = dequant_slice<BITS>(wA[t], make_deq(sA[t], zA[t]), 0);

  auto mfma_slice = [&](const u32x4_t (&a)[kWideMT], const u32x4_t (&b)[2]) {
#pragma unroll
    for (int i = 0; i < kWideMT; ++i)
#pragma unroll
      for (int t = 0; t < 2; ++t) acc[i][t] = mfma32(a[i], b[t], acc[i][t]);
  };
  // Ordering hints for one slice: each MFMA is followed by a few VALU
  // instructions of the next slice's dequantization, and every other one by
  // one of its LDS reads.
  auto interleave = [&]() {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
      __builtin_amdgcn_sched_group_barrier(0x002, wide_valu_per_mfma<BITS>(), 0);   // VALU
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, wide_valu_per_mfma<BITS>(), 0);
    }
  };

  // Step st uses LDS buffer st % 3 and weight set w (wn for step st + 1).
  // On entry a0 / b0 hold slice 0's operands; on exit they hold those of
  // step st + 1 (past the last step: discarded reads of valid memory).
  int bcur = 0;
  auto step = [&](int st, Chunk<BITS> (&w)[2], float (&sw)[2], uint32_t (&zw)[2],
                  const Chunk<BITS> (&wn)[2], const float (&swn)[2], const uint32_t (&zwn)[2]) {
    const int bnext = bcur == 2 ? 0 : bcur + 1, bfill = bnext == 2 ? 0 : bnext + 1;
    const int n2 = min(st + 2, steps - 1);   // past the end: reload the last step (discarded)
    // Each slice is its own scheduling region (sched_barrier), so the
    // interleaving hints see exactly one slice's MFMAs and the work that
    // produces the next slice's operands, and nothing that waits on younger
    // loads is hoisted into an earlier slice.
    load_x(n2, xr);
    Deq d[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) d[t] = make_deq(sw[t], zw[t]);
    // slice 0: produce slice 1
    read_a(bcur, 1, a1);
#pragma unroll
    for (int t = 0; t < 2; ++t) b1[t] = dequant_slice<BITS>(w[t], d[t], 1);
    mfma_slice(a0, b0);
    interleave();
    __builtin_amdgcn_sched_barrier(0);
    // slice 1: produce slice 2
    read_a(bcur, 2, a0);
#pragma unroll
    for (int t = 0; t < 2; ++t) b0[t] = dequant_slice<BITS>(w[t], d[t], 2);
    mfma_slice(a1, b1);
    interleave();
    __builtin_amdgcn_sched_barrier(0);
    // slice 2: produce slice 3; then this step's chunks are free for step st + 2
    read_a(bcur, 3, a1);
#pragma unroll
    for (int t = 0; t < 2; ++t) b1[t] = dequant_slice<BITS>(w[t], d[t], 3);
    mfma_slice(a0, b0);
    interleave();
    load_w(n2, w, sw, zw);
    __builtin_amdgcn_sched_barrier(0);
    // slice 3: produce slice 0 of step st + 1 (its buffer was filled two steps
    // ago, its weights one step ago)
    Deq dn[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) dn[t] = make_deq(swn[t], zwn[t]);
    read_a(bnext, 0, a0);
#pragma unroll
    for (int t = 0; t < 2; ++t) b0[t] = dequant_slice<BITS>(wn[t], dn[t], 0);
    mfma_slice(a1, b1);
    interleave();
    store_x(bfill, xr);
    __syncthreads();
    bcur = bnext;
  };
  for (int st = 0; st < steps; st += 2) {
    step(st, wA, sA, zA, wB, sB, zB);
    step(st + 1, wB, sB, zB, wA, sA, zA);
  }

#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int n = n0 + 32 * t + c32;
    if (n >= N) continue;
#pragma unroll
    for (int i = 0; i < kWideMT; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + 32 * i + 8 * (e / 4) + 4 * h + (e % 4);
        if (m < M) out[(int64_t)m * N + n] = acc[i][t][e];
      }
  }
}

// y = sum of the split partial tiles, in split order (deterministic).
template <bool VEC>
__global__ __launch_bounds__(256) void gemm_split_reduce_kernel(const float *__restrict__ part,
                                                               int64_t mn, int split,
                                                               float *__restrict__ y) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * (VEC ? 4 : 1);
  if (i >= mn) return;
  if constexpr (VEC) {   // mn % 4 == 0: every split's partial is 16-byte aligned
    float4 acc = *reinterpret_cast<const float4 *>(part + i);
    for (int z = 1; z < split; ++z) {
      const float4 v = *reinterpret_cast<const float4 *>(part + (int64_t)z * mn + i);
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
    *reinterpret_cast<float4 *>(y + i) = acc;
  } else {
    float acc = part[i];
    for (int z = 1; z < split; ++z) acc += part[(int64_t)z * mn + i];
    y[i] = acc;
  }
}

template <auto Kernel>
hipError_t set_lds(size_t bytes) {
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void *>(Kernel), hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (attr != hipSuccess) (void)hipGetLastError();   // leave no sticky error behind
  return attr;
}

template <int BITS, bool CM>
hipError_t gemm_bits(const uint16_t *x, const uint32_t *codes, const void *scales,
                     const uint8_t *zeros, int64_t m, int64_t n, int64_t k, float *y, void *ws,
                     hipStream_t st) {
  const GemmPlan plan = gemm_plan(m, n, k);
  if (plan.wide) {
    const hipError_t attr = set_lds<&gemm_wide_kernel<BITS, CM>>(kWideLdsBytes);
    if (attr != hipSuccess) return attr;
    if (plan.split == 1) {
      // row chunks of at most kMaxGridY tiles (the grid's y limit)
      for (int64_t r0 = 0; r0 < m; r0 += kMaxGridY * kWideBM) {
        const int64_t mc = std::min<int64_t>(m - r0, kMaxGridY * kWideBM);
        const dim3 grid((unsigned)((n + kWideBN - 1) / kWideBN), (unsigned)((mc + kWideBM - 1) / kWideBM));
        hipLaunchKernelGGL((gemm_wide_kernel<BITS, CM>), grid, dim3(kThreads), kWideLdsBytes, st,
                           x + r0 * k, codes, scales, zeros, (int)mc, (int)n, (int)k, plan.ksteps,
                           y + r0 * n, nullptr);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
      }
      return hipSuccess;
    }
    // split k: fewer than 256 tiles, so far fewer than kMaxGridY row tiles
    float *part = reinterpret_cast<float *>(static_cast<char *>(ws) + kGemmPartOffset);
    const dim3 grid((unsigned)((n + kWideBN - 1) / kWideBN), (unsigned)((m + kWideBM - 1) / kWideBM),
                    (unsigned)plan.split);
    hipLaunchKernelGGL((gemm_wide_kernel<BITS, CM>), grid, dim3(kThreads), kWideLdsBytes, st, x,
                       codes, scales, zeros, (int)m, (int)n, (int)k, plan.ksteps, y, part);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    const int64_t mn = m * n;
    if (mn % 4 == 0)
      hipLaunchKernelGGL((gemm_split_reduce_kernel<true>), dim3((unsigned)((mn / 4 + 255) / 256)),
                         dim3(256), 0, st, part, mn, plan.split, y);
    else
      hipLaunchKernelGGL((gemm_split_reduce_kernel<false>), dim3((unsigned)((mn + 255) / 256)),
                         dim3(256), 0, st, part, mn, plan.split, y);
    return hipGetLastError();
  }
  const hipError_t attr = set_lds<&gemm_kernel<BITS, CM>>(kLdsBytes);
  if (attr != hipSuccess) return attr;
  const dim3 grid((unsigned)((n + kBN - 1) / kBN), (unsigned)((m + kBM - 1) / kBM));
  hipLaunchKernelGGL((gemm_kernel<BITS, CM>), grid, dim3(kThreads), kLdsBytes, st, x, codes, scales,
                     zeros, (int)m, (int)n, (int)k, y);
  return hipGetLastError();
}

}  // namespace

#ifndef SLQ_GEMM_WIDE_MIN_TILES
#define SLQ_GEMM_WIDE_MIN_TILES 256
#endif
#ifndef SLQ_GEMM_SPLIT_MIN_M
#define SLQ_GEMM_SPLIT_MIN_M 1024
#endif
#ifndef SLQ_GEMM_MAX_SPLIT
#define SLQ_GEMM_MAX_SPLIT 8
#endif
// Wide tiles hold one workgroup per CU, so they need a grid that fills the
// chip.  Smaller grids with many rows split k over the grid's z dimension
// (fp32 partial tiles in the workspace, then one in-order sum); the rest keep
// the 128-row tiles (two workgroups per CU).
GemmPlan gemm_plan(int64_t m, int64_t n, int64_t k) {
  GemmPlan p{false, 1, 0};
  const int64_t tiles = ((n + kWideBN - 1) / kWideBN) * ((m + kWideBM - 1) / kWideBM);
  const int64_t steps = k / kBK;
  if (tiles >= SLQ_GEMM_WIDE_MIN_TILES) {
    p.wide = true;
    p.ksteps = (int)steps;
    return p;
  }
  if (m < SLQ_GEMM_SPLIT_MIN_M || steps < 4) return p;
  int64_t split = std::min<int64_t>({(int64_t)SLQ_GEMM_MAX_SPLIT,
                                     (SLQ_GEMM_WIDE_MIN_TILES + tiles - 1) / tiles, steps / 2});
  const int64_t ksteps = 2 * ((steps + 2 * split - 1) / (2 * split));   // even, >= 2
  split = (steps + ksteps - 1) / ksteps;                                // no empty split
  if (split < 2) return p;
  p.wide = true;
  p.split = (int)split;
  p.ksteps = (int)ksteps;
  return p;
}

size_t gemm_workspace(int64_t m, int64_t n, int64_t k, int) {
  const GemmPlan p = gemm_plan(m, n, k);
  return p.split > 1 ? kGemmPartOffset + (size_t)p.split * m * n * sizeof(float) : 0;
}

hipError_t launch_gemm(const uint16_t *x, const uint32_t *codes, const void *scales,
                       const uint8_t *zeros, bool compact, int64_t m, int64_t n, int64_t k,
                       int bits, float *y, void *ws, hipStream_t s) {
#define SLQ_GEMM_BITS(B_)                                                        \
  case B_:                                                                       \
    return compact ? gemm_bits<B_, true>(x, codes, scales, zeros, m, n, k, y, ws, s) \
                   : gemm_bits<B_, false>(x, codes, scales, zeros, m, n, k, y, ws, s);
  switch (bits) {
    SLQ_GEMM_BITS(2)
    SLQ_GEMM_BITS(3)
    SLQ_GEMM_BITS(4)
    SLQ_GEMM_BITS(5)
    SLQ_GEMM_BITS(6)
    SLQ_GEMM_BITS(7)
    SLQ_GEMM_BITS(8)
    default: return hipErrorInvalidValue;
  }
#undef SLQ_GEMM_BITS
}

}  // namespace slq
