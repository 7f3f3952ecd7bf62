// Decode-path weight-only dequantize matmul (m <= 64) for gfx950.
//
// y[m][n] = sum_g s[n][g] * sum_{k in g} x[m][k] * (q[n][k] - z[n][g])
// (gist.science summary "Statistically-Lossless Quantization of Large Language
// Models", Methodology 3 and Inference Speedup: low-bit group-quantized
// weights against 16-bit activations; SLQ README, Usage 4: weights stored at
// their per-layer bit-width).
//
// The weight stream is the only large operand, so the kernel is bound by HBM
// bandwidth on packed bytes.  Design:
//  * A wavefront owns NT tiles of 16 weight rows and a range of 128-groups.
//    Each lane loads one 32-code chunk (`bits` consecutive words) per row and
//    group, so the 4 lanes of a row read the group's 16*bits bytes contiguously.
//  * Unpacking: two codes are placed in the two 16-bit halves of a register
//    and OR-ed with 0x4300 (bf16 128.0, whose ulp is 1), giving the exact bf16
//    pair (128 + q_a, 128 + q_b) in one shift + one and-or.  Widths that do not
//    divide 16 (3, 5, 6, 7) pair code j with code j+16 of the chunk: both sit
//    at the same offset of their half-stream, so one byte-permute interleaves
//    the half-streams and one shift + and-or extracts each pair; codes that
//    cross a 16-bit boundary are funnel-shifted individually.  8-bit codes are
//    converted exactly (q <= 255 fits bf16's 8 significant bits) with no offset.
//  * MACs run on bf16 MFMA 16x16x32 (x as the 16-row A operand, dequantized
//    weights as B), fp32 accumulate, one chain of 4 MFMAs per group.
//  * Offset and zero point are removed per group in fp32:
//       t = (C - S) - z * S / 128,  S = MFMA chain of x against bf16 128.0
//    S runs the exact instruction sequence C runs for an all-zero group, so
//    C - S is exactly 0 there and (q - z) enters exactly; t is scaled by s
//    with one fma into the fp32 accumulator.
//  * Split-K across workgroups writes fp32 partials; the last workgroup of
//    each row block (atomic ticket, agent-scope release/acquire) sums them in
//    split order, so results are deterministic, and resets its ticket.
#include <algorithm>

#include "launch.h"
#include "slq_device.h"

namespace slq {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr uint32_t kMagic2 = 0x43004300u;   // bf16 pair (128.0, 128.0)
constexpr uint32_t kOne2 = 0x3F803F80u;     // bf16 pair (1.0, 1.0)

// Pair j (0..15) of a 32-code chunk holds codes (c0(j), c1(j)).
template <int BITS>
__host__ __device__ constexpr int pair_c0(int j) {
  return BITS == 2 ? 16 * (j / 8) + (j % 8)
       : BITS == 4 ? 8 * (j / 4) + (j % 4)
       : BITS == 8 ? 2 * j
                   : j;
}
template <int BITS>
__host__ __device__ constexpr int pair_c1(int j) {
  return BITS == 2 ? 16 * (j / 8) + (j % 8) + 8
       : BITS == 4 ? 8 * (j / 4) + (j % 4) + 4
       : BITS == 8 ? 2 * j + 1
                   : j + 16;
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

// 32 codes -> 16 bf16 pairs in pair order (see pair_c0/pair_c1).
template <int BITS>
__device__ __forceinline__ void unpack_pairs(const Chunk<BITS> &c, uint32_t (&p)[16]) {
  if constexpr (BITS == 2) {
#pragma unroll
    for (int d = 0; d < 2; ++d)
#pragma unroll
      for (int i = 0; i < 8; ++i) p[8 * d + i] = ((c.w[d] >> (2 * i)) & 0x00030003u) | kMagic2;
  } else if constexpr (BITS == 4) {
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int i = 0; i < 4; ++i) p[4 * d + i] = ((c.w[d] >> (4 * i)) & 0x000F000Fu) | kMagic2;
  } else if constexpr (BITS == 8) {
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const uint32_t w = c.w[d];
      const uint32_t f0 = __float_as_uint((float)(w & 0xFFu));
      const uint32_t f1 = __float_as_uint((float)((w >> 8) & 0xFFu));
      const uint32_t f2 = __float_as_uint((float)((w >> 16) & 0xFFu));
      const uint32_t f3 = __float_as_uint((float)(w >> 24));
      p[2 * d + 0] = perm(f1, f0, halves_sel(1, 1));
      p[2 * d + 1] = perm(f3, f2, halves_sel(1, 1));
    }
  } else {
    constexpr uint32_t mb = (1u << BITS) - 1u;
    constexpr uint32_t m2 = mb | (mb << 16);
    // W[h] = half-word h of the first half-stream | half-word h of the second.
    uint32_t W[BITS];
#pragma unroll
    for (int h = 0; h < BITS; ++h)
      W[h] = perm(c.w[(BITS + h) / 2], c.w[h / 2], halves_sel(h % 2, (BITS + h) % 2));
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int bit = j * BITS, h = bit / 16, o = bit % 16;
      if (o + BITS <= 16) {
        p[j] = ((W[h] >> o) & m2) | kMagic2;
      } else {
        const int d0 = bit / 32;
        const uint32_t lo = alignbit(c.w[d0 + 1], c.w[d0], bit % 32) & mb;
        const int hb = 16 * BITS + bit, d1 = hb / 32;
        const uint32_t nxt = (d1 + 1 < BITS) ? c.w[d1 + 1] : 0u;
        const uint32_t hi = alignbit(nxt, c.w[d1], hb % 32) & mb;
        p[j] = (lo | (hi << 16)) | kMagic2;
      }
    }
  }
}

// The bf16 pair of activations matching weight pair j.
template <int BITS>
__device__ __forceinline__ uint32_t x_pair(const uint32_t (&X)[16], int j) {
  const int a = pair_c0<BITS>(j), b = pair_c1<BITS>(j);
  if (b == a + 1 && (a % 2) == 0) return X[a / 2];
  return perm(X[b / 2], X[a / 2], halves_sel(a % 2, b % 2));
}

template <int BITS, int MT, int NT>
__global__ __launch_bounds__(kThreads) void gemv_kernel(
    const uint16_t *__restrict__ x, const uint32_t *__restrict__ codes,
    const float *__restrict__ scales, const uint8_t *__restrict__ zeros, int M, int N, int K,
    int ksplits, float *__restrict__ y, float *__restrict__ partial,
    unsigned *__restrict__ tickets) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int col = lane & 15, kq = lane >> 4;
  const int G = K / kGroup;
  const int split = blockIdx.y;
  const int g0 = (int)((int64_t)split * G / ksplits);
  const int g1 = (int)((int64_t)(split + 1) * G / ksplits);
  const int nbase = blockIdx.x * (kWaves * 16 * NT) + wave * (16 * NT);
  const int64_t wpr = (int64_t)K * BITS / 32;   // words per row

  const uint32_t *crow[NT];
  const float *srow[NT];
  const uint8_t *zrow[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int n = min(nbase + 16 * t + col, N - 1);   // rows past N are read, never stored
    crow[t] = codes + (int64_t)n * wpr + kq * BITS;
    srow[t] = scales + (int64_t)n * G;
    zrow[t] = zeros + (int64_t)n * G;
  }
  const uint16_t *xrow[MT];
  bool xvalid[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = 16 * mt + col;
    xvalid[mt] = m < M;
    xrow[mt] = x + (int64_t)(xvalid[mt] ? m : 0) * K + kq * 32;
  }

  f32x4_t acc[NT][MT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[t][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const u32x4_t unit = (BITS == 8) ? u32x4_t{kOne2, kOne2, kOne2, kOne2}
                                   : u32x4_t{kMagic2, kMagic2, kMagic2, kMagic2};

  struct Loads {
    Chunk<BITS> c[NT];
    float s[NT];
    uint32_t z[NT];
    uint32_t X[MT][16];
  };
  auto issue = [&](int g, Loads &L) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      L.c[t] = load_chunk<BITS>(crow[t] + (int64_t)g * 4 * BITS);
      L.s[t] = srow[t][g];
      L.z[t] = zrow[t][g];
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if (xvalid[mt]) {
        const u32x4_t *px = reinterpret_cast<const u32x4_t *>(xrow[mt] + (int64_t)g * kGroup);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const u32x4_t v = px[i];
          L.X[mt][4 * i + 0] = v[0];
          L.X[mt][4 * i + 1] = v[1];
          L.X[mt][4 * i + 2] = v[2];
          L.X[mt][4 * i + 3] = v[3];
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) L.X[mt][i] = 0u;
      }
    }
  };

  Loads cur, nxt;
  if (g0 < g1) issue(g0, cur);
  for (int g = g0; g < g1; ++g) {
    if (g + 1 < g1) issue(g + 1, nxt);

    u32x4_t A[MT][4];
    f32x4_t S[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        A[mt][r] = u32x4_t{x_pair<BITS>(cur.X[mt], 4 * r + 0), x_pair<BITS>(cur.X[mt], 4 * r + 1),
                           x_pair<BITS>(cur.X[mt], 4 * r + 2), x_pair<BITS>(cur.X[mt], 4 * r + 3)};
      S[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int r = 0; r < 4; ++r) S[mt] = mfma16(A[mt][r], unit, S[mt]);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      uint32_t p[16];
      unpack_pairs<BITS>(cur.c[t], p);
      const float s = cur.s[t];
      const float zf = (float)cur.z[t];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        f32x4_t C = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < 4; ++r)
          C = mfma16(A[mt][r], u32x4_t{p[4 * r], p[4 * r + 1], p[4 * r + 2], p[4 * r + 3]}, C);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          float tv;
          if constexpr (BITS == 8) {
            tv = fmaf(-zf, S[mt][v], C[v]);
          } else {
            tv = fmaf(-zf * 0.0078125f, S[mt][v], C[v] - S[mt][v]);
          }
          acc[t][mt][v] = fmaf(s, tv, acc[t][mt][v]);
        }
      }
    }
    if (g + 1 < g1) cur = nxt;
  }

  // Lane holds y rows m = 16*mt + 4*kq + v, column n = nbase + 16*t + col.
  if (ksplits == 1) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int n = nbase + 16 * t + col;
      if (n >= N) continue;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int m = 16 * mt + 4 * kq + v;
          if (m < M) y[(int64_t)m * N + n] = acc[t][mt][v];
        }
    }
    return;
  }

  float *mypart = partial + (int64_t)split * M * N;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int n = nbase + 16 * t + col;
    if (n >= N) continue;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = 16 * mt + 4 * kq + v;
        if (m < M) mypart[(int64_t)m * N + n] = acc[t][mt][v];
      }
  }
  __threadfence();
  __syncthreads();
  __shared__ unsigned last;
  if (threadIdx.x == 0) {
    const unsigned ticket = __hip_atomic_fetch_add(&tickets[blockIdx.x], 1u, __ATOMIC_ACQ_REL,
                                                   __HIP_MEMORY_SCOPE_AGENT);
    last = (ticket == (unsigned)ksplits - 1u);
  }
  __syncthreads();
  if (!last) return;
  __threadfence();
  const int rows = kWaves * 16 * NT;
  const int n0 = blockIdx.x * rows;
  for (int i = threadIdx.x; i < M * rows; i += kThreads) {
    const int m = i / rows, n = n0 + i % rows;
    if (n >= N) continue;
    float sum = 0.f;
    for (int sp = 0; sp < ksplits; ++sp) sum += partial[((int64_t)sp * M + m) * N + n];
    y[(int64_t)m * N + n] = sum;
  }
  if (threadIdx.x == 0)
    __hip_atomic_store(&tickets[blockIdx.x], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

constexpr int kNT = 2;   // 16-row tiles per wavefront
// Split-K tickets live in a fixed area at the start of the workspace, so no
// call's partial sums ever overlap another call's tickets; every completed
// call leaves all tickets at zero.
constexpr size_t kTicketBytes = 65536;
constexpr int64_t kMaxTicketBlocks = kTicketBytes / sizeof(unsigned);

template <int BITS, int MT>
hipError_t gemv_launch(const uint16_t *x, const uint32_t *codes, const float *scales,
                       const uint8_t *zeros, int64_t m, int64_t n, int64_t k, float *y, void *ws,
                       const GemvPlan &plan, hipStream_t st) {
  float *partial = nullptr;
  unsigned *tickets = nullptr;
  if (plan.ksplits > 1) {
    tickets = static_cast<unsigned *>(ws);
    partial = reinterpret_cast<float *>(static_cast<char *>(ws) + kTicketBytes);
  }
  hipLaunchKernelGGL((gemv_kernel<BITS, MT, kNT>), dim3(plan.nblocks, plan.ksplits),
                     dim3(kThreads), 0, st, x, codes, scales, zeros, (int)m, (int)n, (int)k,
                     plan.ksplits, y, partial, tickets);
  return hipGetLastError();
}

template <int BITS>
hipError_t gemv_bits(const uint16_t *x, const uint32_t *codes, const float *scales,
                     const uint8_t *zeros, int64_t m, int64_t n, int64_t k, float *y, void *ws,
                     const GemvPlan &plan, hipStream_t st) {
  switch (plan.mt) {
    case 1: return gemv_launch<BITS, 1>(x, codes, scales, zeros, m, n, k, y, ws, plan, st);
    case 2: return gemv_launch<BITS, 2>(x, codes, scales, zeros, m, n, k, y, ws, plan, st);
    case 3: return gemv_launch<BITS, 3>(x, codes, scales, zeros, m, n, k, y, ws, plan, st);
    case 4: return gemv_launch<BITS, 4>(x, codes, scales, zeros, m, n, k, y, ws, plan, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

GemvPlan gemv_plan(int64_t m, int64_t n, int64_t k, int bits) {
  (void)bits;
  GemvPlan p;
  p.mt = (int)((m + 15) / 16);
  const int64_t rows = kWaves * 16 * kNT;
  p.nblocks = (int)((n + rows - 1) / rows);
  const int64_t G = k / kGroup;
  // Enough workgroups to cover 256 CUs about twice, at least 2 groups per
  // split, and partial sums kept small next to the weight bytes.
  int64_t ks = (512 + p.nblocks - 1) / p.nblocks;
  ks = std::min<int64_t>(ks, std::max<int64_t>(1, G / 2));
  ks = std::min<int64_t>(ks, 16);
  if (p.nblocks > kMaxTicketBlocks) ks = 1;
  p.ksplits = (int)std::max<int64_t>(1, ks);
  if (p.ksplits > 1) {
    p.ws_bytes = kTicketBytes + (size_t)p.ksplits * m * n * sizeof(float);
  } else {
    p.ws_bytes = 0;
  }
  return p;
}

hipError_t launch_gemv(const uint16_t *x, const uint32_t *codes, const float *scales,
                       const uint8_t *zeros, int64_t m, int64_t n, int64_t k, int bits, float *y,
                       void *ws, const GemvPlan &plan, hipStream_t s) {
  switch (bits) {
    case 2: return gemv_bits<2>(x, codes, scales, zeros, m, n, k, y, ws, plan, s);
    case 3: return gemv_bits<3>(x, codes, scales, zeros, m, n, k, y, ws, plan, s);
    case 4: return gemv_bits<4>(x, codes, scales, zeros, m, n, k, y, ws, plan, s);
    case 5: return gemv_bits<5>(x, codes, scales, zeros, m, n, k, y, ws, plan, s);
    case 6: return gemv_bits<6>(x, codes, scales, zeros, m, n, k, y, ws, plan, s);
    case 7: return gemv_bits<7>(x, codes, scales, zeros, m, n, k, y, ws, plan, s);
    case 8: return gemv_bits<8>(x, codes, scales, zeros, m, n, k, y, ws, plan, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace slq
