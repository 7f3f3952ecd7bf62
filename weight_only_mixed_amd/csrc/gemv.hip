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
//  * Offset and zero point, one m-tile (m <= 16): a second chain runs x
//    against the bf16 pair the codes would unpack to if all were equal to z
//    (128 + z, or z for 8 bits), so t = C - S' = x . (q - z) exactly for an
//    all-zero group and for one-hot x; t is scaled by s with one fma.
//    Several m-tiles share one chain of x against bf16 128.0 (or 1.0) per
//    m-tile: t = (C - S) - z * S / 128 (or C - z * S).
//  * x of the workgroup's k-block is staged once in LDS in fragment order.
//    Scales and zero points are staged per wave (each wave reads only its own
//    groups), issued together with the first two weight batches so their HBM
//    round trip overlaps them, in a [group][row] layout whose 16-row reads are
//    bank-conflict free.
//  * Split-K across workgroups writes fp32 partials with device-coherent
//    stores; the last workgroup of each row block (relaxed atomic ticket after
//    the stores have completed) sums them in split order, so results are
//    deterministic, and resets its ticket.  Every access to the partials is an
//    agent-scope atomic: the stores are written through to the device's
//    coherence point and the kernel waits for their completion before taking
//    the ticket, and the last workgroup's loads read from that point, so no
//    cache of another chiplet can hold a stale copy.  The formal form, an
//    acquire-release ticket, adds an L2 writeback and invalidate per workgroup
//    and measured 0.3-7 us slower per launch.
//  * Four kernels: `gemv_kernel` (any m, the general form above),
//    `gemv_tile_kernel` (17..64 rows on large layers: 64 weight rows x 32 or 48
//    activation rows per wavefront, every load reading whole cache-line
//    segments), `gemv_rows_kernel` (33..64 rows on other wide or deep layers:
//    the waves split rows and share each group's activations) and
//    `gemv_mk_kernel` (33..64 rows on mid-width layers: the same sharing with
//    the offset chain formed once per workgroup); the planner at the end of
//    this file picks one.

#include <algorithm>
#include <limits>

#include "launch.h"
#include "slq_device.h"

namespace slq {
namespace {

#ifndef SLQ_GEMV_THREADS
#define SLQ_GEMV_THREADS 256
#endif
constexpr int kThreads = SLQ_GEMV_THREADS;
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

typedef uint32_t u32x4a_t __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x3a_t __attribute__((ext_vector_type(3), aligned(4)));
typedef uint32_t u32x2a_t __attribute__((ext_vector_type(2), aligned(4)));

// One 32-code chunk (BITS words, 4-byte aligned) in as few vector loads as the
// width allows: 4-word parts, then a 3-, 2- or 1-word rest.  The four lanes of
// a row then read its 16*BITS bytes of a group in the same instructions, so
// each load touches one or two 64-byte segments per row: what bounds these
// kernels is the L1's rate of about one segment lookup per cycle.
template <int BITS>
__device__ __forceinline__ Chunk<BITS> load_chunk(const uint32_t *__restrict__ p) {
  Chunk<BITS> c;
#pragma unroll
  for (int i = 0; i + 4 <= BITS; i += 4) {
    const u32x4a_t v = *reinterpret_cast<const u32x4a_t *>(p + i);
    c.w[i] = v[0];
    c.w[i + 1] = v[1];
    c.w[i + 2] = v[2];
    c.w[i + 3] = v[3];
  }
  constexpr int i0 = BITS / 4 * 4;
  if constexpr (BITS % 4 == 3) {
    const u32x3a_t v = *reinterpret_cast<const u32x3a_t *>(p + i0);
    c.w[i0] = v[0];
    c.w[i0 + 1] = v[1];
    c.w[i0 + 2] = v[2];
  } else if constexpr (BITS % 4 == 2) {
    const u32x2a_t v = *reinterpret_cast<const u32x2a_t *>(p + i0);
    c.w[i0] = v[0];
    c.w[i0 + 1] = v[1];
  } else if constexpr (BITS % 4 == 1) {
    c.w[i0] = p[i0];
  }
  return c;
}

// 32 codes -> 16 bf16 pairs in pair order (see pair_c0/pair_c1); `magic` is
// kMagic2 held in a register.
template <int BITS>
__device__ __forceinline__ void unpack_pairs(const Chunk<BITS> &c, uint32_t (&p)[16],
                                             uint32_t magic) {
  if constexpr (BITS == 2) {
#pragma unroll
    for (int d = 0; d < 2; ++d)
#pragma unroll
      for (int i = 0; i < 8; ++i) p[8 * d + i] = ((c.w[d] >> (2 * i)) & 0x00030003u) | magic;
  } else if constexpr (BITS == 4) {
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int i = 0; i < 4; ++i) p[4 * d + i] = ((c.w[d] >> (4 * i)) & 0x000F000Fu) | magic;
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
        p[j] = ((W[h] >> o) & m2) | magic;
      } else {
        const int d0 = bit / 32;
        const uint32_t lo = alignbit(c.w[d0 + 1], c.w[d0], bit % 32) & mb;
        const int hb = 16 * BITS + bit, d1 = hb / 32;
        const uint32_t nxt = (d1 + 1 < BITS) ? c.w[d1 + 1] : 0u;
        const uint32_t hi = alignbit(nxt, c.w[d1], hb % 32) & mb;
        p[j] = (lo | (hi << 16)) | magic;
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

// Activation fragments for one 32-code chunk in pair order: 4 MFMA A operands
// of 4 bf16 pairs each (16 words).
template <int BITS>
__device__ __forceinline__ void x_fragments(const uint32_t (&X)[16], uint32_t (&F)[16]) {
#pragma unroll
  for (int j = 0; j < 16; ++j) F[j] = x_pair<BITS>(X, j);
}

// Split-k tail, run by the last workgroup of a row block: y[m][n0 + r] for
// r < rows is the sum of the k-blocks' partials, added in k-block order.  Each
// thread keeps E outputs x B partial loads in flight (relaxed device-scope
// loads, coherent across XCDs) per round; a chain of dependent loads per
// output had made this tail the longest part of a decode call with many rows.
template <int E, int B>
__device__ __forceinline__ void reduce_partials_eb(const float *__restrict__ partial,
                                                   float *__restrict__ y, int M, int N, int n0,
                                                   int rows, int ksplits, int nthreads) {
  const int total = M * rows;
  const int64_t st = (int64_t)M * N;   // floats per k-block
  for (int i0 = threadIdx.x; i0 < total; i0 += E * nthreads) {
    int64_t off[E];
    bool ok[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int i = i0 + e * nthreads;
      const int m = i / rows, n = n0 + i % rows;
      ok[e] = i < total && n < N;
      off[e] = ok[e] ? (int64_t)m * N + n : 0;
    }
    float sum[E];
#pragma unroll
    for (int e = 0; e < E; ++e) sum[e] = 0.f;
    for (int sp0 = 0; sp0 < ksplits; sp0 += B) {
      float v[E][B];
#pragma unroll
      for (int e = 0; e < E; ++e)
#pragma unroll
        for (int j = 0; j < B; ++j)
          v[e][j] = __hip_atomic_load(partial + off[e] + (int64_t)min(sp0 + j, ksplits - 1) * st,
                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
      for (int e = 0; e < E; ++e)
#pragma unroll
        for (int j = 0; j < B; ++j)
          if (sp0 + j < ksplits) sum[e] += v[e][j];
    }
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (ok[e]) y[off[e]] = sum[e];
  }
}

// gemv_kernel (small register budgets: a wider round measured slower there,
// through occupancy): 4 outputs x 8 splits per round.
__device__ __forceinline__ void reduce_partials(const float *__restrict__ partial,
                                                float *__restrict__ y, int M, int N, int n0,
                                                int rows, int ksplits, int nthreads) {
  reduce_partials_eb<4, 8>(partial, y, M, N, n0, rows, ksplits, nthreads);
}

// The 64-row-tile kernels (rows, mk, tile): a tail of 64 rows x up to 64
// outputs takes one round of up to 64 loads per thread when there are few
// splits (a round is a memory round trip; the summation order is the same, so
// results do not change).  q/o at M = 64: 18.7 -> 16.2 us.
__device__ __forceinline__ void reduce_partials_wide(const float *__restrict__ partial,
                                                     float *__restrict__ y, int M, int N, int n0,
                                                     int rows, int ksplits, int nthreads) {
  if (ksplits <= 2) reduce_partials_eb<32, 2>(partial, y, M, N, n0, rows, ksplits, nthreads);
  else if (ksplits <= 4) reduce_partials_eb<16, 4>(partial, y, M, N, n0, rows, ksplits, nthreads);
  else reduce_partials_eb<8, 8>(partial, y, M, N, n0, rows, ksplits, nthreads);
}

// Workgroup: 4 wavefronts on the same 16*NT rows, each taking a contiguous
// quarter of the workgroup's k-block.  The activations of the k-block are
// staged once in LDS, already permuted into MFMA fragment order, and so are
// the rows' scales and zero points for the k-block.  Each wave streams its
// groups in batches of B with the next batch's loads issued before the
// current batch is consumed (two register buffers), so every lane keeps up to
// 2*B*NT chunk loads in flight.  The first two batches are issued before the
// metadata staging waits, so its HBM round trip overlaps theirs.  The four
// partial sums meet in LDS; with several k-blocks the workgroup partials go to
// the workspace and the last workgroup of each row block adds them in k-block
// order.
template <int BITS, int MT, int NT, int B, bool XD>
struct Batch {
  Chunk<BITS> c[B][NT];
  u32x4_t xv[XD ? B : 1][XD ? MT : 1][4];   // XD: the lane's 32 activations per m-tile and group
};

// Zero-point operand for the single-m-tile kernels: the bf16 pair the codes
// of a group with zero point z would unpack to when all are equal to z
// (128 + z for the offset widths, z itself for 8 bits).  An MFMA chain of x
// against it runs the same instructions as the code chain, so C - S' is
// exactly 0 for an all-zero group and exactly x . (q - z) for one-hot x.
template <int BITS>
__device__ __forceinline__ uint32_t zero_pair(uint32_t z) {
  if constexpr (BITS == 8) return (__float_as_uint((float)z) >> 16) * 0x10001u;
  else return kMagic2 | (z * 0x10001u);
}

// What the metadata area holds next to each scale: the zero-point pair's bits
// (single m-tile) or the zero point as a float.
template <int BITS, bool ZS>
__device__ __forceinline__ float meta_zero(uint32_t z) {
  if constexpr (ZS) return __uint_as_float(zero_pair<BITS>(z));
  else return (float)z;
}

// Metadata staging with MV: one float4 of scales and one u32 of zero points
// (4 consecutive groups of a row) per lane and round; a wave stages its own
// 16*NT rows x [ga, gz) groups.
constexpr int kMetaRounds = 2;
// Without MV, on row blocks of 32 or 64 rows: per-group entries, the first
// kMetaPre rounds per lane loaded ahead of the first weight batches (any
// further rounds after them, one at a time).
#ifndef SLQ_GEMV_META_PRE
#define SLQ_GEMV_META_PRE 4
#endif
constexpr int kMetaPre = SLQ_GEMV_META_PRE;

template <int BITS, int MT, int NT, int B, bool MV, bool XD, int WV, bool CM>
__global__ __launch_bounds__(WV * kWave) void gemv_kernel(
    const uint16_t *__restrict__ x, const uint32_t *__restrict__ codes,
    const void *__restrict__ scales, const uint8_t *__restrict__ zeros, int M, int N, int K,
    int GW, int ksplits, float *__restrict__ y, float *__restrict__ partial,
    unsigned *__restrict__ tickets) {
  // One m-tile: the zero point is folded into a per-row S' chain (see
  // zero_pair); several m-tiles share one S chain per m-tile instead.
  constexpr bool ZS = (MT == 1);
  const MetaRd<BITS, CM> md{scales, zeros};
  extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int col = lane & 15, kq = lane >> 4;
  const int G = K / kGroup;
  const int kb = blockIdx.y;
  const int gbase = kb * GW;
  const int gcount = min(GW, G - gbase);        // groups in this k-block
  const int xpitch = gcount * 64 + 4;           // words per activation row (+16 B vs bank conflicts)
  const int n0 = blockIdx.x * 16 * NT;
  const int64_t wpr = (int64_t)K * BITS / 32;

  // this wave's local group range [ga, gz): a balanced share of the k-block
  // in units of 4 groups (MV) or single groups
  const int gunit = MV ? 4 : 1;
  const int units = gcount / gunit;
  const int ga = (wave * units / WV) * gunit, gz = ((wave + 1) * units / WV) * gunit;

  // ---- stage activations [M][gcount*128] into LDS in fragment order ----
  // (an L2-resident operand: the barrier after it is a short wait).  XD: each
  // lane loads its own activation chunk with the weight batches instead.
  for (int i = threadIdx.x; !XD && i < M * gcount * 4; i += WV * kWave) {
    const int m = i / (gcount * 4), c = i % (gcount * 4);
    const u32x4_t *src =
        reinterpret_cast<const u32x4_t *>(x + (int64_t)m * K + (int64_t)gbase * kGroup + 32 * c);
    uint32_t X[16], F[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x4_t v = src[q];
      X[4 * q + 0] = v[0];
      X[4 * q + 1] = v[1];
      X[4 * q + 2] = v[2];
      X[4 * q + 3] = v[3];
    }
    x_fragments<BITS>(X, F);
    u32x4_t *dst = reinterpret_cast<u32x4_t *>(lds + m * xpitch + c * 16);
#pragma unroll
    for (int r = 0; r < 4; ++r) dst[r] = u32x4_t{F[4 * r], F[4 * r + 1], F[4 * r + 2], F[4 * r + 3]};
  }
  if constexpr (!XD) __syncthreads();   // activations staged

  // ---- scales and zero points: meta[group][16*NT rows] (a tile's 16 rows of
  // one group are 32 consecutive words: conflict-free), each wave stages its own
  // groups [ga, gz), so no workgroup barrier waits on this HBM round trip ----
  float2 *meta = reinterpret_cast<float2 *>(lds + (XD ? 0 : M * xpitch));
  const int mrows = 16 * NT;
  float4 msv[kMetaRounds];
  uint32_t mzv[kMetaRounds];
  const int q4 = (gz - ga) / 4;                  // float4 units per row (MV)
  const int munits = mrows * q4;                 // <= kWave * kMetaRounds (planned)
  if constexpr (MV) {
    if (munits > 0) {
#pragma unroll
      for (int r = 0; r < kMetaRounds; ++r) {
        const int e = min(lane + r * kWave, munits - 1);
        const int n = min(n0 + e / q4, N - 1);
        const int64_t o = (int64_t)n * G + gbase + ga + 4 * (e % q4);
        md.load4(o, msv[r], mzv[r]);
      }
    }
  }
  // Without MV, entry i is (row i / cnt, group ga + i % cnt).  Wide row
  // blocks (PRE): the first kMetaPre rounds are loaded with the first weight
  // batches, ahead of them, and stored after them; returns come back in issue
  // order, so the stores wait for these loads alone.  (A loop that stored each
  // entry as it arrived made one memory round trip per round before the first
  // weight load; on 16-row blocks, whose waves stage one round or two, that
  // loop measured faster.)
  constexpr bool PRE = !MV && NT > 1 && WV <= 8;   // (16-wave instances have no registers to spare)
  const int cnt = gz - ga;
  const int mtot = MV ? 0 : mrows * cnt;
  if constexpr (!MV && !PRE) {
    for (int i = lane; i < mtot; i += kWave) {
      const int n = min(n0 + i / cnt, N - 1);
      const int gl = ga + i % cnt;
      const int64_t o = (int64_t)n * G + gbase + gl;
      meta[gl * mrows + i / cnt] = make_float2(md.scale(o), meta_zero<BITS, ZS>(md.zero(o)));
    }
  }
  float psv[PRE ? kMetaPre : 1];
  uint32_t pzv[PRE ? kMetaPre : 1];

  const uint32_t *crow[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int n = min(n0 + 16 * t + col, N - 1);   // rows past N are read, never stored
    crow[t] = codes + (int64_t)n * wpr + (int64_t)gbase * 4 * BITS + kq * BITS;
  }
  // Loads past the wave's last group are skipped (a wave-uniform branch):
  // reloading the last group instead kept the two buffers' instruction shape
  // but cost a wait for redundant loads before the reduction barrier.
  // XD: rows min(16 mt + col, M-1) of x, this lane's 32-value chunk of each group
  const u32x4_t *xrow[XD ? MT : 1];
#pragma unroll
  for (int mt = 0; mt < (XD ? MT : 1); ++mt)
    xrow[mt] = reinterpret_cast<const u32x4_t *>(x + (int64_t)min(16 * mt + col, M - 1) * K +
                                                 (int64_t)gbase * kGroup + 32 * kq);
  auto load = [&](Batch<BITS, MT, NT, B, XD> &bt, int g) {
#pragma unroll
    for (int j = 0; j < B; ++j) {
      if (g + j >= gz) break;   // past the wave's last group: nothing to wait for at the end
      const int gg = g + j;
      if constexpr (XD) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int q = 0; q < 4; ++q) bt.xv[j][mt][q] = xrow[mt][gg * (kGroup / 8) + q];
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) bt.c[j][t] = load_chunk<BITS>(crow[t] + (int64_t)gg * 4 * BITS);
    }
  };

  const uint32_t magic = in_vgpr(kMagic2);
  const uint32_t unit1 = (BITS == 8) ? kOne2 : kMagic2;
  const u32x4_t unit = u32x4_t{unit1, unit1, unit1, unit1};
  f32x4_t acc[NT][MT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[t][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const Batch<BITS, MT, NT, B, XD> &bt, int g) {
#pragma unroll
    for (int j = 0; j < B; ++j) {
      const int gl = g + j;
      if (gl >= gz) break;
      // x fragments; rows past M repeat row M-1 and only feed unstored outputs
      u32x4_t A[MT][4];
      if constexpr (XD) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          uint32_t X[16], F[16];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            X[4 * q + 0] = bt.xv[j][mt][q][0];
            X[4 * q + 1] = bt.xv[j][mt][q][1];
            X[4 * q + 2] = bt.xv[j][mt][q][2];
            X[4 * q + 3] = bt.xv[j][mt][q][3];
          }
          x_fragments<BITS>(X, F);
#pragma unroll
          for (int r = 0; r < 4; ++r)
            A[mt][r] = u32x4_t{F[4 * r], F[4 * r + 1], F[4 * r + 2], F[4 * r + 3]};
        }
      } else {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const int m = min(16 * mt + col, M - 1);
          const u32x4_t *src =
              reinterpret_cast<const u32x4_t *>(lds + m * xpitch + (gl * 4 + kq) * 16);
#pragma unroll
          for (int r = 0; r < 4; ++r) A[mt][r] = src[r];
        }
      }
      f32x4_t S[MT];
      if constexpr (!ZS) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          S[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int r = 0; r < 4; ++r) S[mt] = mfma16(A[mt][r], unit, S[mt]);
        }
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        uint32_t p[16];
        unpack_pairs<BITS>(bt.c[j][t], p, magic);
        const float2 sz = meta[gl * (16 * NT) + 16 * t + col];
        const float s = sz.x;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          f32x4_t C = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int r = 0; r < 4; ++r)
            C = mfma16(A[mt][r], u32x4_t{p[4 * r], p[4 * r + 1], p[4 * r + 2], p[4 * r + 3]}, C);
          if constexpr (ZS) {
            const uint32_t zp = __float_as_uint(sz.y);
            const u32x4_t zb = u32x4_t{zp, zp, zp, zp};
            f32x4_t Z = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int r = 0; r < 4; ++r) Z = mfma16(A[mt][r], zb, Z);
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[t][mt][v] = fmaf(s, C[v] - Z[v], acc[t][mt][v]);
          } else {
            const float zf = sz.y;
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
      }
    }
  };

  // Ring of two batch buffers: both are filled before the staging barrier, and
  // each is refilled (two batches ahead) as soon as it has been consumed.
  // PRE: the metadata loads share the weight batches' branch (on a path
  // without the batches, the compiler's in-order wait counts would have to
  // assume nothing in flight behind them, and the stores would wait for
  // every load).
  Batch<BITS, MT, NT, B, XD> b0, b1;
  if (ga < gz) {
    if constexpr (PRE) {
#pragma unroll
      for (int u = 0; u < kMetaPre; ++u) {
        const int i = min(lane + u * kWave, mtot - 1);   // clamped: no load is skipped
        const int n = min(n0 + i / cnt, N - 1);
        const int64_t o = (int64_t)n * G + gbase + ga + i % cnt;
        psv[u] = md.scale(o);
        pzv[u] = md.zero(o);
      }
    }
    load(b0, ga);
    load(b1, ga + B);
  }
  if constexpr (PRE) {
#pragma unroll
    for (int u = 0; u < kMetaPre; ++u) {
      const int i = lane + u * kWave;
      if (i < mtot) meta[(ga + i % cnt) * mrows + i / cnt] = make_float2(psv[u], meta_zero<BITS, ZS>(pzv[u]));
    }
    for (int i = lane + kMetaPre * kWave; i < mtot; i += kWave) {
      const int n = min(n0 + i / cnt, N - 1);
      const int gl = ga + i % cnt;
      const int64_t o = (int64_t)n * G + gbase + gl;
      meta[gl * mrows + i / cnt] = make_float2(md.scale(o), meta_zero<BITS, ZS>(md.zero(o)));
    }
  }
  if constexpr (MV) {
#pragma unroll
    for (int r = 0; r < kMetaRounds; ++r) {
      const int e = lane + r * kWave;
      if (e < munits) {
        const int base = (ga + 4 * (e % q4)) * mrows + e / q4;
        meta[base + 0 * mrows] = make_float2(msv[r].x, meta_zero<BITS, ZS>(mzv[r] & 0xFFu));
        meta[base + 1 * mrows] = make_float2(msv[r].y, meta_zero<BITS, ZS>((mzv[r] >> 8) & 0xFFu));
        meta[base + 2 * mrows] = make_float2(msv[r].z, meta_zero<BITS, ZS>((mzv[r] >> 16) & 0xFFu));
        meta[base + 3 * mrows] = make_float2(msv[r].w, meta_zero<BITS, ZS>(mzv[r] >> 24));
      }
    }
  }
  // the wave's own metadata writes precede its reads in LDS program order
  if (ga < gz) {
    for (int g = ga;;) {
      compute(b0, g);
      load(b0, g + 2 * B);
      g += B;
      if (g >= gz) break;
      compute(b1, g);
      load(b1, g + 2 * B);
      g += B;
      if (g >= gz) break;
    }
  }

  // ---- reduce the WV waves' partials in LDS (reusing the activation area) ----
  __syncthreads();
  f32x4_t *red = reinterpret_cast<f32x4_t *>(lds);
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) red[((wave * NT + t) * MT + mt) * kWave + lane] = acc[t][mt];
  __syncthreads();
  // wave w sums the (t, mt) tiles with (t * MT + mt) % WV == w, adding waves in order
  for (int e = wave; e < NT * MT; e += WV) {
    const int t = e / MT, mt = e % MT;
    f32x4_t sum = red[(t * MT + mt) * kWave + lane];
#pragma unroll
    for (int w = 1; w < WV; ++w) sum += red[((w * NT + t) * MT + mt) * kWave + lane];
    const int n = n0 + 16 * t + col;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = 16 * mt + 4 * kq + v;
      if (m >= M || n >= N) continue;
      if (ksplits == 1) {
        y[(int64_t)m * N + n] = sum[v];
      } else {
        // device-scope store: coherent across XCDs without an L2 writeback
        __hip_atomic_store(&partial[((int64_t)kb * M + m) * N + n], sum[v], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  if (ksplits == 1) return;
  // every partial store has completed (device scope) before the ticket is taken
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  __shared__ unsigned last;
  if (threadIdx.x == 0) {
    const unsigned ticket = __hip_atomic_fetch_add(&tickets[blockIdx.x], 1u, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
    last = (ticket == (unsigned)ksplits - 1u);
  }
  __syncthreads();
  if (!last) return;
  reduce_partials(partial, y, M, N, n0, 16 * NT, ksplits, WV * kWave);
  if (threadIdx.x == 0)
    __hip_atomic_store(&tickets[blockIdx.x], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Decode with 33..64 activation rows on wide or deep layers (mid-width layers
// take gemv_mk_kernel instead).  The activations of a group (up to
// 64 x 128 bf16) are the large operand next to a 16-row weight tile, so the
// four wavefronts of a workgroup split rows instead of k: wavefront w owns
// rows [16w, 16w + 16) of the workgroup's 64, and all four read one copy of
// each group's activations, staged in LDS in fragment order (double buffered,
// one barrier per group; the loads of group g+2 are issued during group g).
// Each wavefront keeps kRowsDepth groups of its codes in flight and stages
// its rows' scales and zero points for the k-block in LDS.  Zero points use
// one shared S chain per m-tile (t = (C - S) - z * S / 128, or C - z * S).
#ifndef SLQ_GEMV_ROWS_DEPTH
#define SLQ_GEMV_ROWS_DEPTH 4
#endif
constexpr int kRowsDepth = SLQ_GEMV_ROWS_DEPTH;
constexpr int kRowsXPitch = 68;   // words per activation row and group (64 + 4 vs bank conflicts)

template <int BITS, int MT, bool CM>
__global__ __launch_bounds__(kThreads) void gemv_rows_kernel(
    const uint16_t *__restrict__ x, const uint32_t *__restrict__ codes,
    const void *__restrict__ scales, const uint8_t *__restrict__ zeros, int M, int N, int K,
    int GW, int ksplits, float *__restrict__ y, float *__restrict__ partial,
    unsigned *__restrict__ tickets) {
  const MetaRd<BITS, CM> md{scales, zeros};
  static_assert(kThreads == 256, "four wavefronts of 16 rows");
  extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int col = lane & 15, kq = lane >> 4;
  const int G = K / kGroup;
  const int kb = blockIdx.y;
  const int gbase = kb * GW;
  const int gcount = min(GW, G - gbase);
  const int nw = blockIdx.x * 64 + 16 * wave;   // this wave's first row
  const int64_t wpr = (int64_t)K * BITS / 32;

  uint32_t *xbuf[2] = {lds, lds + M * kRowsXPitch};
  float2 *meta = reinterpret_cast<float2 *>(lds + 2 * M * kRowsXPitch) + wave * gcount * 16;

  // activation staging: thread t owns chunk t % 4 of row t / 4 (clamped past M)
  const int xm = min((int)threadIdx.x / 4, M - 1), xc = threadIdx.x % 4;
  const bool xowner = (int)threadIdx.x < 4 * M;
  const u32x4_t *xsrc =
      reinterpret_cast<const u32x4_t *>(x + (int64_t)xm * K + (int64_t)gbase * kGroup + 32 * xc);
  auto xload = [&](int g, u32x4_t (&v)[4]) {
    const int gg = min(g, gcount - 1);
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = xsrc[gg * (kGroup / 8) + q];
  };
  auto xstore = [&](uint32_t *buf, const u32x4_t (&v)[4]) {
    if (!xowner) return;
    uint32_t X[16], F[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      X[4 * q + 0] = v[q][0];
      X[4 * q + 1] = v[q][1];
      X[4 * q + 2] = v[q][2];
      X[4 * q + 3] = v[q][3];
    }
    x_fragments<BITS>(X, F);
    u32x4_t *dst = reinterpret_cast<u32x4_t *>(buf + xm * kRowsXPitch + xc * 16);
#pragma unroll
    for (int q = 0; q < 4; ++q) dst[q] = u32x4_t{F[4 * q], F[4 * q + 1], F[4 * q + 2], F[4 * q + 3]};
  };

  const uint32_t *crow = codes + (int64_t)min(nw + col, N - 1) * wpr + (int64_t)gbase * 4 * BITS + kq * BITS;
  auto cload = [&](int g) { return load_chunk<BITS>(crow + (int64_t)min(g, gcount - 1) * 4 * BITS); };

  // prologue: x(0), the code ring, x(1), then this wave's metadata
  u32x4_t xr0[4], xr1[4];
  xload(0, xr0);
  Chunk<BITS> ring[kRowsDepth];
#pragma unroll
  for (int d = 0; d < kRowsDepth; ++d) ring[d] = cload(d);
  xload(1, xr1);
  for (int i = lane; i < 16 * gcount; i += kWave) {
    const int r = i / gcount, gl = i % gcount;
    const int64_t o = (int64_t)min(nw + r, N - 1) * G + gbase + gl;
    meta[gl * 16 + r] = make_float2(md.scale(o), (float)md.zero(o));
  }
  xstore(xbuf[0], xr0);
  __syncthreads();

  const uint32_t magic = in_vgpr(kMagic2);
  const uint32_t unit1 = (BITS == 8) ? kOne2 : kMagic2;
  const u32x4_t unit = u32x4_t{unit1, unit1, unit1, unit1};
  f32x4_t acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // group g: x(g) is in xbuf[g % 2]; x(g+1) waits in register set (g+1) % 2
  auto body = [&](int g, const Chunk<BITS> &c, u32x4_t (&xfree)[4], const u32x4_t (&xnext)[4]) {
    xload(g + 2, xfree);
    const uint32_t *buf = xbuf[g & 1];
    u32x4_t A[MT][4];
    f32x4_t S[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = min(16 * mt + col, M - 1);
      const u32x4_t *src = reinterpret_cast<const u32x4_t *>(buf + m * kRowsXPitch + kq * 16);
#pragma unroll
      for (int r = 0; r < 4; ++r) A[mt][r] = src[r];
      S[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int r = 0; r < 4; ++r) S[mt] = mfma16(A[mt][r], unit, S[mt]);
    }
    uint32_t p[16];
    unpack_pairs<BITS>(c, p, magic);
    const float2 sz = meta[g * 16 + col];
    const float s = sz.x, zf = sz.y;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      f32x4_t C = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int r = 0; r < 4; ++r)
        C = mfma16(A[mt][r], u32x4_t{p[4 * r], p[4 * r + 1], p[4 * r + 2], p[4 * r + 3]}, C);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float tv;
        if constexpr (BITS == 8) tv = fmaf(-zf, S[mt][v], C[v]);
        else tv = fmaf(-zf * 0.0078125f, S[mt][v], C[v] - S[mt][v]);
        acc[mt][v] = fmaf(s, tv, acc[mt][v]);
      }
    }
    if (g + 1 < gcount) xstore(xbuf[(g + 1) & 1], xnext);
    __syncthreads();
  };

  for (int g0 = 0; g0 < gcount; g0 += kRowsDepth) {
#pragma unroll
    for (int j = 0; j < kRowsDepth; ++j) {
      const int g = g0 + j;
      if (g >= gcount) break;
      if (j % 2 == 0) body(g, ring[j], xr0, xr1);
      else body(g, ring[j], xr1, xr0);
      if (g + kRowsDepth < gcount) ring[j] = cload(g + kRowsDepth);
    }
  }

  // ---- outputs: rows nw + col, m = 16 mt + 4 kq + v ----
  const int n = nw + col;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = 16 * mt + 4 * kq + v;
      if (m >= M || n >= N) continue;
      if (ksplits == 1) y[(int64_t)m * N + n] = acc[mt][v];
      else
        __hip_atomic_store(&partial[((int64_t)kb * M + m) * N + n], acc[mt][v], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
  if (ksplits == 1) return;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  __shared__ unsigned last;
  if (threadIdx.x == 0) {
    const unsigned ticket = __hip_atomic_fetch_add(&tickets[blockIdx.x], 1u, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
    last = (ticket == (unsigned)ksplits - 1u);
  }
  __syncthreads();
  if (!last) return;
  reduce_partials_wide(partial, y, M, N, blockIdx.x * 64, 64, ksplits, kThreads);
  if (threadIdx.x == 0)
    __hip_atomic_store(&tickets[blockIdx.x], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Several m-tiles on mid-width layers: `gemv_mk_kernel`.
// The four wavefronts of a workgroup work on the same group at a time, each on
// its own NT tiles of 16 weight rows (64*NT rows per workgroup), so one LDS copy
// of a group's activations serves all of them and every A operand read from
// LDS feeds NT MFMA chains.  The offset chain S = x . 128 (x . 1 for 8 bits)
// does not depend on the weight row: it is formed once per workgroup and group,
// by wavefront mt for m-tile mt, one group ahead, and shared through LDS.  It is
// the same MFMA instruction sequence as a code chain on all-zero codes, so
// C - S is exactly 0 for an all-zero group.  Activations pass through three LDS
// buffers (the current group's, the next group's, from which S is formed, and
// the one being written), with one barrier per group.  Each lane keeps
// kMkDepth groups of its codes, scales and zero points in flight in registers.
#ifndef SLQ_GEMV_MK_DEPTH
#define SLQ_GEMV_MK_DEPTH 2
#endif
constexpr int kMkDepth = SLQ_GEMV_MK_DEPTH;
static_assert(kMkDepth % 2 == 0, "activation register sets alternate per group");

template <int BITS, int NT>
struct MkSlot {
  Chunk<BITS> c[NT];
  float s[NT];
  uint32_t z[NT];
};

template <int BITS, int MT, int NT, bool CM>
__global__ __launch_bounds__(kThreads) void gemv_mk_kernel(
    const uint16_t *__restrict__ x, const uint32_t *__restrict__ codes,
    const void *__restrict__ scales, const uint8_t *__restrict__ zeros, int M, int N, int K,
    int GW, int ksplits, float *__restrict__ y, float *__restrict__ partial,
    unsigned *__restrict__ tickets) {
  static_assert(kThreads == 256 && MT <= kWaves, "four wavefronts, one per S m-tile");
  constexpr int RW = 16 * NT;           // weight rows per wavefront
  constexpr int RB = kWaves * RW;       // weight rows per workgroup
  const MetaRd<BITS, CM> md{scales, zeros};
  extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int col = lane & 15, kq = lane >> 4;
  const int G = K / kGroup;
  const int kb = blockIdx.y;
  const int gbase = kb * GW;
  const int gcount = min(GW, G - gbase);
  const int nw = blockIdx.x * RB + RW * wave;   // this wave's first row
  const int64_t wpr = (int64_t)K * BITS / 32;
  const int xw = M * kRowsXPitch;               // words per activation buffer
  float *sbuf = reinterpret_cast<float *>(lds + 3 * xw);   // [2][16 * MT]
  auto xbuf = [&](int g) { return lds + (g % 3) * xw; };

  // activation staging: thread t owns chunk t % 4 of row t / 4 (clamped past M)
  const int xm = min((int)threadIdx.x / 4, M - 1), xc = threadIdx.x % 4;
  const bool xowner = (int)threadIdx.x < 4 * M;
  const u32x4_t *xsrc =
      reinterpret_cast<const u32x4_t *>(x + (int64_t)xm * K + (int64_t)gbase * kGroup + 32 * xc);
  auto xload = [&](int g, u32x4_t (&v)[4]) {
    const int gg = min(g, gcount - 1);
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = xsrc[gg * (kGroup / 8) + q];
  };
  auto xstore = [&](uint32_t *buf, const u32x4_t (&v)[4]) {
    if (!xowner) return;
    uint32_t X[16], F[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      X[4 * q + 0] = v[q][0];
      X[4 * q + 1] = v[q][1];
      X[4 * q + 2] = v[q][2];
      X[4 * q + 3] = v[q][3];
    }
    x_fragments<BITS>(X, F);
    u32x4_t *dst = reinterpret_cast<u32x4_t *>(buf + xm * kRowsXPitch + xc * 16);
#pragma unroll
    for (int q = 0; q < 4; ++q) dst[q] = u32x4_t{F[4 * q], F[4 * q + 1], F[4 * q + 2], F[4 * q + 3]};
  };

  // codes, scale and zero point of this lane's rows for group g
  const uint32_t *crow[NT];
  int64_t mrow[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int64_t r = min(nw + 16 * t + col, N - 1);
    crow[t] = codes + r * wpr + (int64_t)gbase * 4 * BITS + kq * BITS;
    mrow[t] = r * G + gbase;
  }
  auto sload = [&](int g, MkSlot<BITS, NT> &o) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      o.c[t] = load_chunk<BITS>(crow[t] + (int64_t)g * 4 * BITS);
      o.s[t] = md.scale(mrow[t] + g);
      o.z[t] = md.zero(mrow[t] + g);
    }
  };

  const uint32_t unit1 = (BITS == 8) ? kOne2 : kMagic2;
  const u32x4_t unit = u32x4_t{unit1, unit1, unit1, unit1};
  // S of group g for m-tile `wave`, from its activation buffer
  auto s_chain = [&](int g) {
    if (wave >= MT) return;
    const int m = min(16 * wave + col, M - 1);
    const u32x4_t *src = reinterpret_cast<const u32x4_t *>(xbuf(g) + m * kRowsXPitch + kq * 16);
    f32x4_t S = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 4; ++r) S = mfma16(src[r], unit, S);
    if (col == 0) *reinterpret_cast<f32x4_t *>(sbuf + (g & 1) * 16 * MT + 16 * wave + 4 * kq) = S;
  };

  // prologue: x(0), x(1) staged; x(2), x(3) in registers; the code ring; S(0)
  u32x4_t xr[2][4];
  xload(0, xr[0]);
  xload(1, xr[1]);
  MkSlot<BITS, NT> ring[kMkDepth];
  // (loads are unconditional, clamped to the last group, so the number of
  // loads in flight is the same on every path and the waits stay partial)
#pragma unroll
  for (int d = 0; d < kMkDepth; ++d) sload(min(d, gcount - 1), ring[d]);
  xstore(xbuf(0), xr[0]);
  xstore(xbuf(1), xr[1]);
  xload(2, xr[0]);
  xload(3, xr[1]);
  __syncthreads();
  s_chain(0);
  __syncthreads();

  const uint32_t magic = in_vgpr(kMagic2);
  f32x4_t acc[NT][MT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[t][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // group g: x(g) in buffer g % 3, x(g + 1) in buffer (g + 1) % 3 (both
  // published), S(g) in sbuf[g & 1]; x(g + 2) waits in xs and goes to buffer
  // (g + 2) % 3, which was last read before the previous barrier.
  auto body = [&](int g, const MkSlot<BITS, NT> &c, u32x4_t (&xs)[4]) {
    if (g + 1 < gcount) s_chain(g + 1);
    const uint32_t *buf = xbuf(g);
    uint32_t p[NT][16];
#pragma unroll
    for (int t = 0; t < NT; ++t) unpack_pairs<BITS>(c.c[t], p[t], magic);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = min(16 * mt + col, M - 1);
      const u32x4_t *src = reinterpret_cast<const u32x4_t *>(buf + m * kRowsXPitch + kq * 16);
      u32x4_t A[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) A[r] = src[r];
      const f32x4_t S = *reinterpret_cast<const f32x4_t *>(sbuf + (g & 1) * 16 * MT + 16 * mt + 4 * kq);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        f32x4_t C = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < 4; ++r)
          C = mfma16(A[r], u32x4_t{p[t][4 * r], p[t][4 * r + 1], p[t][4 * r + 2], p[t][4 * r + 3]}, C);
        const float zf = (float)c.z[t];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          float tv;
          if constexpr (BITS == 8) tv = fmaf(-zf, S[v], C[v]);
          else tv = fmaf(-zf * 0.0078125f, S[v], C[v] - S[v]);
          acc[t][mt][v] = fmaf(c.s[t], tv, acc[t][mt][v]);
        }
      }
    }
    // buffer (g + 2) % 3 is read by no one in this step; past the end it
    // receives a copy of the last group that is never used
    xstore(xbuf(g + 2), xs);
    xload(g + 4, xs);
    __syncthreads();
  };

  // whole blocks of kMkDepth groups (no exit inside, so every trip leaves the
  // same loads in flight), then the remaining groups, already in the ring
  const int nfull = gcount / kMkDepth;
  for (int it = 0; it < nfull; ++it) {
#pragma unroll
    for (int j = 0; j < kMkDepth; ++j) {
      const int g = it * kMkDepth + j;
      body(g, ring[j], xr[j % 2]);
      sload(min(g + kMkDepth, gcount - 1), ring[j]);
    }
  }
#pragma unroll
  for (int j = 0; j < kMkDepth - 1; ++j) {
    const int g = nfull * kMkDepth + j;
    if (g >= gcount) break;
    body(g, ring[j], xr[j % 2]);
  }

  // ---- outputs: rows nw + 16 t + col, m = 16 mt + 4 kq + v ----
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int n = nw + 16 * t + col;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = 16 * mt + 4 * kq + v;
        if (m >= M || n >= N) continue;
        if (ksplits == 1) y[(int64_t)m * N + n] = acc[t][mt][v];
        else
          __hip_atomic_store(&partial[((int64_t)kb * M + m) * N + n], acc[t][mt][v],
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
  }
  if (ksplits == 1) return;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  __shared__ unsigned last;
  if (threadIdx.x == 0) {
    const unsigned ticket = __hip_atomic_fetch_add(&tickets[blockIdx.x], 1u, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
    last = (ticket == (unsigned)ksplits - 1u);
  }
  __syncthreads();
  if (!last) return;
  reduce_partials_wide(partial, y, M, N, blockIdx.x * RB, RB, ksplits, kThreads);
  if (threadIdx.x == 0)
    __hip_atomic_store(&tickets[blockIdx.x], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// 17..64 activation rows: `gemv_tile_kernel`.
// A wavefront owns kTileNT tiles of 16 weight rows and MTW m-tiles of 16
// activation rows (2 or 3) over a contiguous share of the workgroup's k-block,
// so each activation fragment feeds kTileNT code chains and each unpacked code
// operand feeds MTW chains.  The four wavefronts of a workgroup split the
// activation rows MS ways and the k-block 4/MS ways; the k shares meet in LDS
// at the end.
// What bounds these kernels is the L1's rate of about one cache-line lookup per
// cycle, not bytes: a load whose 64 lanes each touch another 64-byte segment
// costs 64 lookups.  So every load here reads whole segments:
//  * activations are loaded row-contiguous (16 lanes per 256-byte group row)
//    and transposed to fragment order through a wavefront-private LDS stage;
//  * a lane's 32-code chunk comes in one or two vector loads (load_chunk), so
//    the four lanes of a row read its 16*b bytes in the same instructions;
//  * scales and zero points of the wavefront's groups are staged in LDS once,
//    16 consecutive groups of a row per 4 lanes.
// Codes and activations of the next group are loaded while the current group
// is used (two register slots, unconditional clamped loads in whole slot
// pairs, scheduling fences keeping each slot's loads after the body that
// frees it).  The offset chain S = x . 128 (x . 1 for 8 bits) is formed per
// wave and group with the same MFMA sequence as a code chain of all-zero
// codes, so an all-zero group adds exactly 0 and one-hot activations give
// w_hat exactly: t = C - (1 + z/128) S (C - z S for 8 bits) with one fma.
#ifndef SLQ_GEMV_TILE_NT
#define SLQ_GEMV_TILE_NT 4
#endif
constexpr int kTileNT = SLQ_GEMV_TILE_NT;
// m-tiles per wavefront: 2 at 17..32 rows and at 49..64 rows (there the
// activation rows are split over two wavefront pairs, so each code is
// unpacked twice); 3 at 33..48 rows, every wavefront on all activation rows
// and its own quarter of the k-block, so each code is unpacked once per
// workgroup.  Measured on the 8B gate/up and down shapes at b = 3, 4, 6, 8:
// 3 m-tiles beat the split pairs by 5-10% at 40 and 48 rows; 4 m-tiles at 64
// rows were 3-10% slower than the split pairs.
constexpr int kTileMTW = 2;
constexpr int kTileMTW3MaxM = 48;
constexpr int kTileMaxGroups = 16;   // groups per wavefront (its metadata stage)
constexpr int kTileXPitch = 68;      // words per staged activation row (64 + 4 against bank conflicts)
#ifndef SLQ_GEMV_TILE_WV
#define SLQ_GEMV_TILE_WV 4
#endif
constexpr int kTileWV = SLQ_GEMV_TILE_WV;   // wavefronts per workgroup
// LDS of a workgroup: per wavefront an activation stage and a metadata stage
// (fp32 scales and byte zero points of kTileMaxGroups groups x 16*kTileNT rows)
constexpr size_t tile_lds_bytes(int wv, int mtw) {
  return (size_t)wv * (16 * mtw * kTileXPitch * 4 + kTileMaxGroups * 16 * kTileNT * 5) + 16;
}

template <int BITS, int MTW>
struct TileSlot {
  Chunk<BITS> c[kTileNT];
  u32x4_t xv[4 * MTW];   // 16 * MTW activation rows x 256 bytes, 16 bytes per lane and load
};

template <int BITS, int MTW, int MS, int WV, bool CM>
__global__ __launch_bounds__(WV * kWave) void gemv_tile_kernel(
    const uint16_t *__restrict__ x, const uint32_t *__restrict__ codes,
    const void *__restrict__ scales, const uint8_t *__restrict__ zeros, int M, int N, int K,
    int GW, int ksplits, float *__restrict__ y, float *__restrict__ partial,
    unsigned *__restrict__ tickets) {
  static_assert(MS == 1 || MS == 2, "WV wavefronts: MS along m, WV / MS along k");
  constexpr int KW = WV / MS;                // wavefronts along k
  constexpr int RB = 16 * kTileNT;           // weight rows per workgroup
  constexpr int NO = kTileNT * MTW * 4;      // outputs per lane
  constexpr int XI = 4 * MTW;                // activation loads per lane and group
  constexpr int XW = 16 * MTW * kTileXPitch; // words of a wavefront's activation stage
  static_assert(RB == kWave, "one staged metadata row per lane");
  static_assert(NO * kWave <= XW, "the k-share partials fit the wavefront's activation stage");
  const MetaRd<BITS, CM> md{scales, zeros};
  extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
  uint32_t *xs_all = lds;                                                   // [WV][XW]
  float *ms_all = reinterpret_cast<float *>(lds + WV * XW);                 // [WV][groups][RB]
  uint8_t *mzz_all = reinterpret_cast<uint8_t *>(ms_all + WV * kTileMaxGroups * RB);
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int ms = wave / KW, kw = wave % KW;
  const int col = lane & 15, kq = lane >> 4;
  const int G = K / kGroup;
  const int kb = blockIdx.y;
  const int gbase = kb * GW;
  const int gcount = min(GW, G - gbase);
  const int ga = (gcount * kw) / KW, gz = (gcount * (kw + 1)) / KW;   // relative to gbase
  const int ng = gz - ga;                                              // <= kTileMaxGroups
  const int n0 = blockIdx.x * RB;
  const int64_t wpr = (int64_t)K * BITS / 32;
  uint32_t *xs = xs_all + wave * XW;
  float *mzs = ms_all + wave * kTileMaxGroups * RB;
  uint8_t *mzz = mzz_all + wave * kTileMaxGroups * RB;

  const uint32_t *crow[kTileNT];
#pragma unroll
  for (int t = 0; t < kTileNT; ++t) {
    const int64_t r = min(n0 + 16 * t + col, N - 1);
    crow[t] = codes + r * wpr + (int64_t)gbase * 4 * BITS + kq * BITS;
  }
  // activation load j covers staged rows 4j .. 4j+3, 16 bytes per lane
  const int prow = lane >> 4, ppc = lane & 15;
  uint32_t xoff[XI];
#pragma unroll
  for (int j = 0; j < XI; ++j) {
    const int m = min(16 * MTW * ms + 4 * j + prow, M - 1);
    xoff[j] = (uint32_t)m * (uint32_t)(K / 8) + (uint32_t)ppc;
  }
  const u32x4_t *xg = reinterpret_cast<const u32x4_t *>(x) + (int64_t)gbase * (kGroup / 8);
  auto load = [&](int g, TileSlot<BITS, MTW> &o) {
#pragma unroll
    for (int t = 0; t < kTileNT; ++t) o.c[t] = load_chunk<BITS>(crow[t] + (int64_t)g * 4 * BITS);
    const u32x4_t *xp = xg + (int64_t)g * (kGroup / 8);
#pragma unroll
    for (int j = 0; j < XI; ++j) o.xv[j] = xp[xoff[j]];
  };

  const uint32_t magic = in_vgpr(kMagic2);
  const uint32_t unit1 = (BITS == 8) ? kOne2 : kMagic2;
  const u32x4_t unit = u32x4_t{unit1, unit1, unit1, unit1};
  f32x4_t acc[kTileNT][MTW];
#pragma unroll
  for (int t = 0; t < kTileNT; ++t)
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt) acc[t][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto body = [&](const TileSlot<BITS, MTW> &sl, int gl) {
    // transpose the activations to fragment order through the wave's stage
#pragma unroll
    for (int j = 0; j < XI; ++j)
      *reinterpret_cast<u32x4_t *>(xs + (4 * j + prow) * kTileXPitch + 4 * ppc) = sl.xv[j];
    u32x4_t A[MTW][4];
    f32x4_t S[MTW];
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt) {
      uint32_t X[16], F[16];
      const u32x4_t *src = reinterpret_cast<const u32x4_t *>(xs + (16 * mt + col) * kTileXPitch + 16 * kq);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x4_t v = src[q];
        X[4 * q + 0] = v[0];
        X[4 * q + 1] = v[1];
        X[4 * q + 2] = v[2];
        X[4 * q + 3] = v[3];
      }
      x_fragments<BITS>(X, F);
#pragma unroll
      for (int r = 0; r < 4; ++r) A[mt][r] = u32x4_t{F[4 * r], F[4 * r + 1], F[4 * r + 2], F[4 * r + 3]};
      S[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int r = 0; r < 4; ++r) S[mt] = mfma16(A[mt][r], unit, S[mt]);
    }
#pragma unroll
    for (int t = 0; t < kTileNT; ++t) {
      uint32_t p[16];
      unpack_pairs<BITS>(sl.c[t], p, magic);
      const float s = mzs[gl * RB + 16 * t + col];
      const float zf = (float)mzz[gl * RB + 16 * t + col];
      const float nz = (BITS == 8) ? -zf : -(1.0f + zf * 0.0078125f);
#pragma unroll
      for (int mt = 0; mt < MTW; ++mt) {
        f32x4_t C = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < 4; ++r)
          C = mfma16(A[mt][r], u32x4_t{p[4 * r], p[4 * r + 1], p[4 * r + 2], p[4 * r + 3]}, C);
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[t][mt][v] = fmaf(s, fmaf(nz, S[mt][v], C[v]), acc[t][mt][v]);
      }
    }
  };

  if (ng > 0) {
    // metadata of the wave's groups: entry (row r, group gl) at [gl * RB + r];
    // lanes 16u .. 16u+15 of load u take 16 consecutive groups of row 4u + lane / 16
    constexpr int MU = kTileMaxGroups * RB / kWave;
    float sv[MU];
    uint32_t zv[MU];
#pragma unroll
    for (int u = 0; u < MU; ++u) {
      const int i = u * kWave + lane;
      const int r = i / kTileMaxGroups, gl = min(i % kTileMaxGroups, ng - 1);
      const int64_t o = (int64_t)min(n0 + r, N - 1) * G + gbase + ga + gl;
      sv[u] = md.scale(o);
      zv[u] = md.zero(o);
    }
    TileSlot<BITS, MTW> sa, sb;
    __builtin_amdgcn_sched_barrier(0);
    load(ga, sa);
    __builtin_amdgcn_sched_barrier(0);
    load(min(ga + 1, gz - 1), sb);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < MU; ++u) {
      const int i = u * kWave + lane;
      const int e = (i % kTileMaxGroups) * RB + i / kTileMaxGroups;
      mzs[e] = sv[u];
      mzz[e] = (uint8_t)zv[u];
    }
    int g = ga;
    for (; g + 2 < gz; g += 2) {
      body(sa, g - ga);
      __builtin_amdgcn_sched_barrier(0);
      load(g + 2, sa);
      __builtin_amdgcn_sched_barrier(0);
      body(sb, g + 1 - ga);
      __builtin_amdgcn_sched_barrier(0);
      load(min(g + 3, gz - 1), sb);
      __builtin_amdgcn_sched_barrier(0);
    }
    body(sa, g - ga);
    if (g + 1 < gz) body(sb, g + 1 - ga);
  }

  // the k shares meet in LDS (each wavefront's own activation stage); wavefront
  // kw = 0 adds them in kw order
  if (kw > 0) {
    float *dst = reinterpret_cast<float *>(xs) + lane;
#pragma unroll
    for (int t = 0; t < kTileNT; ++t)
#pragma unroll
      for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) dst[((t * MTW + mt) * 4 + v) * kWave] = acc[t][mt][v];
  }
  __syncthreads();
  if (kw == 0) {
#pragma unroll
    for (int j = 1; j < KW; ++j) {
      const float *src = reinterpret_cast<const float *>(xs_all + (wave + j) * XW) + lane;
#pragma unroll
      for (int t = 0; t < kTileNT; ++t)
#pragma unroll
        for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[t][mt][v] += src[((t * MTW + mt) * 4 + v) * kWave];
    }
#pragma unroll
    for (int t = 0; t < kTileNT; ++t)
#pragma unroll
      for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int m = 16 * (MTW * ms + mt) + 4 * kq + v, n = n0 + 16 * t + col;
          if (m >= M || n >= N) continue;
          if (ksplits == 1) y[(int64_t)m * N + n] = acc[t][mt][v];
          else
            __hip_atomic_store(&partial[((int64_t)kb * M + m) * N + n], acc[t][mt][v],
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
  }
  if (ksplits == 1) return;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  __shared__ unsigned last;
  if (threadIdx.x == 0) {
    const unsigned ticket = __hip_atomic_fetch_add(&tickets[blockIdx.x], 1u, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
    last = (ticket == (unsigned)ksplits - 1u);
  }
  __syncthreads();
  if (!last) return;
  reduce_partials_wide(partial, y, M, N, n0, RB, ksplits, WV * kWave);
  if (threadIdx.x == 0)
    __hip_atomic_store(&tickets[blockIdx.x], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Split-K tickets live in a fixed area at the start of the workspace, so no
// call's partial sums ever overlap another call's tickets; every completed
// call leaves all tickets at zero.
constexpr size_t kTicketBytes = 65536;
constexpr int64_t kMaxTicketBlocks = kTicketBytes / sizeof(unsigned);

// LDS: the activation tile [m][groups*128] in fragment order, reused for the
// cross-wave reduction.
size_t gemv_lds_bytes(int64_t m, int mt, int nt, int gw, bool xd, int wv) {
  const size_t xs = xd ? 0 : (size_t)m * (gw * 64 + 4) * 4;
  const size_t meta = (size_t)16 * nt * gw * 8;
  const size_t red = (size_t)wv * nt * mt * kWave * 16;
  return std::max(xs + meta, red) + 16;
}
#ifndef SLQ_GEMV_LDS_BUDGET
#define SLQ_GEMV_LDS_BUDGET 65536
#endif
constexpr size_t kLdsBudget = SLQ_GEMV_LDS_BUDGET;   // activation bytes per workgroup
#ifndef SLQ_GEMV_LDS_BUDGET_WIDE
#define SLQ_GEMV_LDS_BUDGET_WIDE 131072
#endif
constexpr size_t kLdsBudgetWide = SLQ_GEMV_LDS_BUDGET_WIDE;   // the same for a workgroup alone on its CU
#ifndef SLQ_GEMV_TARGET_BLOCKS
#define SLQ_GEMV_TARGET_BLOCKS 256
#endif
constexpr int64_t kTargetBlocks = SLQ_GEMV_TARGET_BLOCKS;
#ifndef SLQ_GEMV_TARGET_BLOCKS_TINY
#define SLQ_GEMV_TARGET_BLOCKS_TINY 64
#endif
constexpr int64_t kTargetBlocksTiny = SLQ_GEMV_TARGET_BLOCKS_TINY;
#ifndef SLQ_GEMV_XD_MIN_M
#define SLQ_GEMV_XD_MIN_M 5
#endif
constexpr int64_t kXdMinM = SLQ_GEMV_XD_MIN_M;
#ifndef SLQ_GEMV_XD_MIN_GROUPS
#define SLQ_GEMV_XD_MIN_GROUPS 64
#endif
constexpr int64_t kXdMinGroups = SLQ_GEMV_XD_MIN_GROUPS;
#ifndef SLQ_GEMV_ROWS_MIN_MT
#define SLQ_GEMV_ROWS_MIN_MT 3
#endif
constexpr int kRowsMinMt = SLQ_GEMV_ROWS_MIN_MT;   // fewest m-tiles for the row-split kernel
// gemv_mk_kernel: workgroups aimed for, fewest groups per k-block, and the
// narrowest layer given 128-row workgroups (by default none: 128-row
// workgroups measured slower than 64-row ones on every layer tried).
// It serves layers 2048..8191 wide with 49..64 rows (4 m-tiles), or with
// 33..48 rows (3 m-tiles) when there are at least kMkMinM rows or the layer is
// at least kMkDeepK deep: there it measured 3-11% faster than the
// per-lane-activation and row-split kernels (q/o at 48 and 64 rows, the down
// projection at 40, 48 and 64); on wider and narrower layers, with fewer rows,
// and on q/o at 40 rows those measured faster.
#ifndef SLQ_GEMV_MK_MIN_MT
#define SLQ_GEMV_MK_MIN_MT 3
#endif
constexpr int kMkMinMt = SLQ_GEMV_MK_MIN_MT;
#ifndef SLQ_GEMV_MK_MIN_M
#define SLQ_GEMV_MK_MIN_M 48
#endif
#ifndef SLQ_GEMV_MK_DEEP_K
#define SLQ_GEMV_MK_DEEP_K 8192
#endif
constexpr int64_t kMkMinM = SLQ_GEMV_MK_MIN_M, kMkDeepK = SLQ_GEMV_MK_DEEP_K;
#ifndef SLQ_GEMV_MK_MIN_N
#define SLQ_GEMV_MK_MIN_N 2048
#endif
#ifndef SLQ_GEMV_MK_MAX_N
#define SLQ_GEMV_MK_MAX_N 8191
#endif
constexpr int64_t kMkMinN = SLQ_GEMV_MK_MIN_N, kMkMaxN = SLQ_GEMV_MK_MAX_N;
#ifndef SLQ_GEMV_MK_TARGET
#define SLQ_GEMV_MK_TARGET 256
#endif
constexpr int64_t kMkTarget = SLQ_GEMV_MK_TARGET;
#ifndef SLQ_GEMV_MK_MIN_GROUPS
#define SLQ_GEMV_MK_MIN_GROUPS 4
#endif
constexpr int64_t kMkMinGroups = SLQ_GEMV_MK_MIN_GROUPS;
#ifndef SLQ_GEMV_MK_NT2_MIN_N
#define SLQ_GEMV_MK_NT2_MIN_N (1LL << 40)
#endif
constexpr int64_t kMkNt2MinN = SLQ_GEMV_MK_NT2_MIN_N;
// 17..64 rows: the tile kernel from kTileMinM rows on layers of at least
// kTileMinSize parameters (smaller layers have too few 64-row tiles to fill
// the chip, and the older kernels measured faster there).
#ifndef SLQ_GEMV_TILE_MIN_M
#define SLQ_GEMV_TILE_MIN_M 17
#endif
#ifndef SLQ_GEMV_TILE_MIN_SIZE
#define SLQ_GEMV_TILE_MIN_SIZE (1LL << 25)
#endif
constexpr int64_t kTileMinM = SLQ_GEMV_TILE_MIN_M, kTileMinSize = SLQ_GEMV_TILE_MIN_SIZE;
#ifndef SLQ_GEMV_TILE_MIN_BLOCKS
#define SLQ_GEMV_TILE_MIN_BLOCKS 192
#endif
constexpr int64_t kTileMinBlocks = SLQ_GEMV_TILE_MIN_BLOCKS, kTileFillBlocks = 256;
// Groups per load batch for 1, 2 and 4 row tiles (two batches in flight).
#ifndef SLQ_GEMV_B_NT1
#define SLQ_GEMV_B_NT1 4
#endif
#ifndef SLQ_GEMV_B_NT2
#define SLQ_GEMV_B_NT2 2
#endif
#ifndef SLQ_GEMV_B_NT4
#define SLQ_GEMV_B_NT4 1
#endif
constexpr int kBatchNt1 = SLQ_GEMV_B_NT1, kBatchNt2 = SLQ_GEMV_B_NT2, kBatchNt4 = SLQ_GEMV_B_NT4;
// One m-tile on a grid of at most kWvBlocks workgroups (one per CU or fewer):
// 16 wavefronts per workgroup (8 when activations are loaded per lane, whose
// register footprint would spill at 16) instead of 4, all on the same rows,
// so that each SIMD has several wavefronts to overlap load latency, unpacking
// and MFMA chains.  Larger grids keep 4: wider workgroups would no longer all
// be resident at once.
#ifndef SLQ_GEMV_WV_BLOCKS
#define SLQ_GEMV_WV_BLOCKS 256
#endif
constexpr int64_t kWvBlocks = SLQ_GEMV_WV_BLOCKS;
// Dynamic LDS ceiling per workgroup: activations (<= 64 KiB + pitch padding)
// plus scales/zero points (<= 32 KiB), or the reduction area (<= 64 KiB).
constexpr size_t kMaxDynLds = 152 * 1024;   // activation tile, metadata and the kernel's own LDS stay within 160 KiB

template <int BITS, int MT, int NT, int B, bool MV, bool XD, int WV, bool CM>
hipError_t gemv_launch(const uint16_t *x, const uint32_t *codes, const void *scales,
                       const uint8_t *zeros, int64_t m, int64_t n, int64_t k, float *y, void *ws,
                       const GemvPlan &plan, hipStream_t st) {
  float *partial = nullptr;
  unsigned *tickets = nullptr;
  if (plan.ksplits > 1) {
    tickets = static_cast<unsigned *>(ws);
    partial = reinterpret_cast<float *>(static_cast<char *>(ws) + kTicketBytes);
  }
  const size_t lds = gemv_lds_bytes(m, MT, NT, plan.gw, XD, WV);
  if (lds > kMaxDynLds) return hipErrorInvalidValue;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void *>(&gemv_kernel<BITS, MT, NT, B, MV, XD, WV, CM>),
      hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxDynLds);
  if (attr != hipSuccess) {
    (void)hipGetLastError();   // leave no sticky error behind for later calls
    return attr;
  }
  hipLaunchKernelGGL((gemv_kernel<BITS, MT, NT, B, MV, XD, WV, CM>), dim3(plan.nblocks, plan.ksplits),
                     dim3(WV * kWave), lds, st, x, codes, scales, zeros, (int)m, (int)n, (int)k,
                     plan.gw, plan.ksplits, y, partial, tickets);
  return hipGetLastError();
}

// Groups per load batch: kBatchNt* (NT * B = 4 chunk loads per batch per
// lane by default), two batches in flight.
template <int BITS, int MT, bool CM>
hipError_t gemv_shape(const uint16_t *x, const uint32_t *codes, const void *scales,
                      const uint8_t *zeros, int64_t m, int64_t n, int64_t k, float *y, void *ws,
                      const GemvPlan &plan, hipStream_t st) {
// One m-tile may use 8 waves per workgroup, or 16 with LDS-staged activations
// (more waves on the same rows for occupancy); several m-tiles use 4.
#define SLQ_GEMV_LAUNCH_WV(NT_, B_, MV_, XD_, WV_) \
  gemv_launch<BITS, MT, NT_, B_, MV_, XD_, WV_, CM>(x, codes, scales, zeros, m, n, k, y, ws, plan, st)
#define SLQ_GEMV_LAUNCH(NT_, B_, MV_, XD_)                                                  \
  (MT == 1 && !XD_ && plan.wv == 16                                                         \
       ? SLQ_GEMV_LAUNCH_WV(NT_, B_, MV_, XD_, (MT == 1 && !XD_ ? 16 : 4))                 \
   : MT == 1 && plan.wv == 8 ? SLQ_GEMV_LAUNCH_WV(NT_, B_, MV_, XD_, (MT == 1 ? 8 : 4))     \
                             : SLQ_GEMV_LAUNCH_WV(NT_, B_, MV_, XD_, 4))
// Direct activation loads with several m-tiles hold MT x 16 registers of x
// per group: one group per batch.
#define SLQ_GEMV_NT(NT_, B_)                                                            \
  case NT_:                                                                             \
    if constexpr (NT_ * MT <= 4 || MT == 1) {                                           \
      if (plan.xd) {                                                                    \
        constexpr int BX = MT == 1 ? B_ : 1;                                            \
        return plan.mv ? SLQ_GEMV_LAUNCH(NT_, BX, true, true)                           \
                       : SLQ_GEMV_LAUNCH(NT_, BX, false, true);                         \
      }                                                                                 \
    }                                                                                   \
    if constexpr (MT == 1)                                                              \
      return plan.mv ? SLQ_GEMV_LAUNCH(NT_, B_, true, false)                            \
                     : SLQ_GEMV_LAUNCH(NT_, B_, false, false);                          \
    return hipErrorInvalidValue;
  switch (plan.nt) {
    SLQ_GEMV_NT(1, kBatchNt1)
    SLQ_GEMV_NT(2, kBatchNt2)
    SLQ_GEMV_NT(4, kBatchNt4)
    default: return hipErrorInvalidValue;
  }
#undef SLQ_GEMV_NT
#undef SLQ_GEMV_LAUNCH
#undef SLQ_GEMV_LAUNCH_WV
}

size_t gemv_rows_lds_bytes(int64_t m, int gw) {
  return (size_t)2 * m * kRowsXPitch * 4 + (size_t)kWaves * gw * 16 * 8 + 16;
}

template <int BITS, int MT, bool CM>
hipError_t gemv_rows_launch(const uint16_t *x, const uint32_t *codes, const void *scales,
                            const uint8_t *zeros, int64_t m, int64_t n, int64_t k, float *y,
                            void *ws, const GemvPlan &plan, hipStream_t st) {
  float *partial = nullptr;
  unsigned *tickets = nullptr;
  if (plan.ksplits > 1) {
    tickets = static_cast<unsigned *>(ws);
    partial = reinterpret_cast<float *>(static_cast<char *>(ws) + kTicketBytes);
  }
  const size_t lds = gemv_rows_lds_bytes(m, plan.gw);
  if (lds > kMaxDynLds) return hipErrorInvalidValue;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void *>(&gemv_rows_kernel<BITS, MT, CM>),
      hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxDynLds);
  if (attr != hipSuccess) {
    (void)hipGetLastError();
    return attr;
  }
  hipLaunchKernelGGL((gemv_rows_kernel<BITS, MT, CM>), dim3(plan.nblocks, plan.ksplits),
                     dim3(kThreads), lds, st, x, codes, scales, zeros, (int)m, (int)n, (int)k,
                     plan.gw, plan.ksplits, y, partial, tickets);
  return hipGetLastError();
}

size_t gemv_mk_lds_bytes(int64_t m, int mt) {
  return (size_t)3 * m * kRowsXPitch * 4 + (size_t)2 * 16 * mt * 4 + 16;
}

template <int BITS, int MT, int NT, bool CM>
hipError_t gemv_mk_launch(const uint16_t *x, const uint32_t *codes, const void *scales,
                          const uint8_t *zeros, int64_t m, int64_t n, int64_t k, float *y,
                          void *ws, const GemvPlan &plan, hipStream_t st) {
  float *partial = nullptr;
  unsigned *tickets = nullptr;
  if (plan.ksplits > 1) {
    tickets = static_cast<unsigned *>(ws);
    partial = reinterpret_cast<float *>(static_cast<char *>(ws) + kTicketBytes);
  }
  const size_t lds = gemv_mk_lds_bytes(m, MT);
  if (lds > kMaxDynLds) return hipErrorInvalidValue;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void *>(&gemv_mk_kernel<BITS, MT, NT, CM>),
      hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxDynLds);
  if (attr != hipSuccess) {
    (void)hipGetLastError();
    return attr;
  }
  hipLaunchKernelGGL((gemv_mk_kernel<BITS, MT, NT, CM>), dim3(plan.nblocks, plan.ksplits),
                     dim3(kThreads), lds, st, x, codes, scales, zeros, (int)m, (int)n, (int)k,
                     plan.gw, plan.ksplits, y, partial, tickets);
  return hipGetLastError();
}

template <int BITS, int MT, bool CM>
hipError_t gemv_mk_nt(const uint16_t *x, const uint32_t *codes, const void *scales,
                      const uint8_t *zeros, int64_t m, int64_t n, int64_t k, float *y, void *ws,
                      const GemvPlan &plan, hipStream_t st) {
  if constexpr (kMkNt2MinN < ((int64_t)1 << 40))
    if (plan.nt == 2) return gemv_mk_launch<BITS, MT, 2, CM>(x, codes, scales, zeros, m, n, k, y, ws, plan, st);
  return gemv_mk_launch<BITS, MT, 1, CM>(x, codes, scales, zeros, m, n, k, y, ws, plan, st);
}

template <int BITS, int MTW, int MS, bool CM>
hipError_t gemv_tile_launch(const uint16_t *x, const uint32_t *codes, const void *scales,
                            const uint8_t *zeros, int64_t m, int64_t n, int64_t k, float *y,
                            void *ws, const GemvPlan &plan, hipStream_t st) {
  // every wavefront's share of a k-block must fit its metadata stage
  if ((plan.gw + kTileWV / MS - 1) / (kTileWV / MS) > kTileMaxGroups) return hipErrorInvalidValue;
  constexpr size_t lds = tile_lds_bytes(kTileWV, MTW);
  static_assert(lds <= kMaxDynLds, "tile kernel LDS");
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void *>(&gemv_tile_kernel<BITS, MTW, MS, kTileWV, CM>),
      hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr != hipSuccess) {
    (void)hipGetLastError();
    return attr;
  }
  float *partial = nullptr;
  unsigned *tickets = nullptr;
  if (plan.ksplits > 1) {
    tickets = static_cast<unsigned *>(ws);
    partial = reinterpret_cast<float *>(static_cast<char *>(ws) + kTicketBytes);
  }
  hipLaunchKernelGGL((gemv_tile_kernel<BITS, MTW, MS, kTileWV, CM>), dim3(plan.nblocks, plan.ksplits),
                     dim3(kTileWV * kWave), lds, st, x, codes, scales, zeros, (int)m, (int)n, (int)k,
                     plan.gw, plan.ksplits, y, partial, tickets);
  return hipGetLastError();
}

template <int BITS, bool CM>
hipError_t gemv_bits(const uint16_t *x, const uint32_t *codes, const void *scales,
                     const uint8_t *zeros, int64_t m, int64_t n, int64_t k, float *y, void *ws,
                     const GemvPlan &plan, hipStream_t st) {
  if (plan.tile) {
    if (plan.mtw == 2)
      return plan.ms == 2 ? gemv_tile_launch<BITS, 2, 2, CM>(x, codes, scales, zeros, m, n, k, y, ws, plan, st)
                          : gemv_tile_launch<BITS, 2, 1, CM>(x, codes, scales, zeros, m, n, k, y, ws, plan, st);
    if (plan.mtw == 3)
      return gemv_tile_launch<BITS, 3, 1, CM>(x, codes, scales, zeros, m, n, k, y, ws, plan, st);
    return hipErrorInvalidValue;
  }
  if (plan.mk) {
    // only the m-tile counts and row tiles the planner can choose are built
    switch (plan.mt) {
      case 2:
        if constexpr (kMkMinMt <= 2)
          return gemv_mk_nt<BITS, 2, CM>(x, codes, scales, zeros, m, n, k, y, ws, plan, st);
        return hipErrorInvalidValue;
      case 3:
        if constexpr (kMkMinMt <= 3)
          return gemv_mk_nt<BITS, 3, CM>(x, codes, scales, zeros, m, n, k, y, ws, plan, st);
        return hipErrorInvalidValue;
      case 4: return gemv_mk_nt<BITS, 4, CM>(x, codes, scales, zeros, m, n, k, y, ws, plan, st);
      default: return hipErrorInvalidValue;
    }
  }
  if (plan.rows) {
    switch (plan.mt) {
      case 1: return gemv_rows_launch<BITS, 1, CM>(x, codes, scales, zeros, m, n, k, y, ws, plan, st);
      case 2: return gemv_rows_launch<BITS, 2, CM>(x, codes, scales, zeros, m, n, k, y, ws, plan, st);
      case 3: return gemv_rows_launch<BITS, 3, CM>(x, codes, scales, zeros, m, n, k, y, ws, plan, st);
      case 4: return gemv_rows_launch<BITS, 4, CM>(x, codes, scales, zeros, m, n, k, y, ws, plan, st);
      default: return hipErrorInvalidValue;
    }
  }
  switch (plan.mt) {
    case 1: return gemv_shape<BITS, 1, CM>(x, codes, scales, zeros, m, n, k, y, ws, plan, st);
    case 2: return gemv_shape<BITS, 2, CM>(x, codes, scales, zeros, m, n, k, y, ws, plan, st);
    case 3: return gemv_shape<BITS, 3, CM>(x, codes, scales, zeros, m, n, k, y, ws, plan, st);
    case 4: return gemv_shape<BITS, 4, CM>(x, codes, scales, zeros, m, n, k, y, ws, plan, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

GemvPlan gemv_plan(int64_t m, int64_t n, int64_t k, int bits) {
  (void)bits;
  GemvPlan p{};
  p.mt = (int)((m + 15) / 16);
  const int64_t G = k / kGroup;
  // 33..64 activation rows on a wide or deep layer: the row-split kernel (one
  // LDS copy of each group's activations for 64 weight rows) beats per-lane
  // activation loads, whose L2 traffic grows with n * k * m / 16; narrower
  // layers and 17..32 rows measured faster with per-lane loads.
  p.wv = kWaves;
  if (m >= kTileMinM && n * k >= kTileMinSize) {
    // 17..64 rows on a large layer: gemv_tile_kernel, 16 * kTileNT rows per
    // workgroup, mtw m-tiles per wavefront, the activation rows split
    // kTileWV / kw ways and the k-block kw ways.
    p.tile = true;
    p.wv = kTileWV;
    p.mtw = (m > 16 * kTileMTW && m <= kTileMTW3MaxM) ? 3 : kTileMTW;
    p.ms = (m > 16 * p.mtw) ? 2 : 1;
    p.nt = kTileNT;
    p.b = 2;
    const int64_t kw = kTileWV / p.ms;
    const int64_t nb = (n + 16 * kTileNT - 1) / (16 * kTileNT);
    // k is split across workgroups only as far as a wavefront's metadata
    // stage (kTileMaxGroups groups) requires: splits for occupancy measured
    // slower, their tails (partial sums, ticket, reduction) cost more than
    // the second wavefront per SIMD gains
    int64_t ks = std::max<int64_t>(1, (G + kTileMaxGroups * kw - 1) / (kTileMaxGroups * kw));
    // ... except, when every wavefront covers all activation rows (17..48
    // rows), on grids that would leave a quarter of the CUs idle (the down
    // projection: 64 row tiles x 2 k-blocks), which split k for about 256
    // workgroups while each wavefront keeps 6 groups or more.  (With the
    // activation rows split over wavefront pairs, and so fewer groups per
    // wavefront, such splits measured slower.)
    if (p.ms == 1 && nb * ks < kTileMinBlocks)
      ks = std::max<int64_t>(ks, std::min<int64_t>((kTileFillBlocks + nb - 1) / nb, G / (6 * kw)));
    const int64_t gw = std::max<int64_t>(1, (G + ks - 1) / ks);
    p.gw = (int)std::min<int64_t>(gw, std::numeric_limits<int>::max());
    p.ksplits = (int)((G + gw - 1) / gw);
    p.nblocks = (int)nb;
    if ((p.nblocks > kMaxTicketBlocks && p.ksplits > 1) || (G + gw - 1) / gw > 65535) p.ksplits = 0;
    p.ws_bytes = p.ksplits > 1 ? kTicketBytes + (size_t)p.ksplits * m * n * sizeof(float) : 0;
    return p;
  }
  const bool mk_rows = p.mt >= 4 || (p.mt == 3 && (m >= kMkMinM || k >= kMkDeepK));
  if (p.mt >= kMkMinMt && mk_rows && n >= kMkMinN && n <= kMkMaxN) {
    // 33..64 rows on a mid-width layer: gemv_mk_kernel, one LDS copy of each
    // group's activations for 64*nt rows; k is split only for lack of
    // workgroups, keeping at least kMkMinGroups groups per k-block.
    p.mk = true;
    p.rows = false;
    p.mv = false;
    p.xd = false;
    p.b = kMkDepth;
    p.nt = n >= kMkNt2MinN ? 2 : 1;
    const int64_t rb = 64 * p.nt;
    const int64_t nb = (n + rb - 1) / rb;
    int64_t ks = std::max<int64_t>(1, (kMkTarget + nb - 1) / nb);
    ks = std::min<int64_t>(ks, std::max<int64_t>(1, G / kMkMinGroups));
    const int64_t gw = std::max<int64_t>(1, (G + ks - 1) / ks);
    p.gw = (int)std::min<int64_t>(gw, std::numeric_limits<int>::max());
    p.ksplits = (int)((G + gw - 1) / gw);
    p.nblocks = (int)nb;
    if ((p.nblocks > kMaxTicketBlocks && p.ksplits > 1) || (G + gw - 1) / gw > 65535 ||
        gemv_mk_lds_bytes(m, p.mt) > kMaxDynLds)
      p.ksplits = 0;   // not supported
    p.ws_bytes = p.ksplits > 1 ? kTicketBytes + (size_t)p.ksplits * m * n * sizeof(float) : 0;
    return p;
  }
  p.rows = p.mt >= kRowsMinMt && (n >= 8192 || k >= 8192);
  if (p.rows) {
    // row-split kernel: 64 rows per workgroup; split k only for lack of
    // workgroups, keeping at least 8 groups per k-block
    p.nt = 4;
    p.mv = false;
    p.xd = false;
    p.b = kRowsDepth;
    const int64_t nb = (n + 63) / 64;
    int64_t ks = std::max<int64_t>(1, (kTargetBlocks + nb - 1) / nb);
    ks = std::min<int64_t>(ks, std::max<int64_t>(1, G / 8));
    int64_t gw = (G + ks - 1) / ks;
    gw = std::min<int64_t>(std::max<int64_t>(gw, 1), 64);
    p.gw = (int)gw;
    p.ksplits = (int)((G + gw - 1) / gw);
    p.nblocks = (int)nb;
    if ((p.nblocks > kMaxTicketBlocks && p.ksplits > 1) || p.ksplits > 65535) p.ksplits = 0;
    p.ws_bytes = p.ksplits > 1 ? kTicketBytes + (size_t)p.ksplits * m * n * sizeof(float) : 0;
    return p;
  }
  // Fewest k-blocks such that the activations of a k-block fit the LDS budget
  // and about kTargetBlocks workgroups exist; widest row tiles first (they
  // amortize the activation staging).  Every split adds a partial-sum round
  // trip at the end, so splits are only made for lack of workgroups.
  // One m-tile of more than a few rows on a long k: activations come straight
  // from L2 with the weight batches (no LDS tile, so no LDS bound on the
  // k-block and fewer splits); short k keeps the LDS tile, which measured
  // faster there.
  // Several m-tiles always load x directly: an LDS tile of 17..64 rows would
  // cap the k-block at a few groups and multiply the split-K partial sums.
  p.xd = (p.mt == 1 && m >= kXdMinM && G >= kXdMinGroups) || p.mt > 1;
  const int64_t gw_max =
      p.xd ? std::max<int64_t>(1, G)
           : std::max<int64_t>(1, (int64_t)kLdsBudget / (std::max<int64_t>(m, 1) * 256));
  const int64_t ks_min = std::max<int64_t>(1, (G + gw_max - 1) / gw_max);
  // Tiny activations: splits only for lack of workgroups on narrow layers.
  const int64_t target = m <= 4 ? kTargetBlocksTiny : kTargetBlocks;
  p.nt = 1;
  for (int nt : {4, 2, 1}) {
    if (nt * p.mt > (p.xd && p.mt > 1 ? 4 : 8)) continue;   // register budget
    if (m <= 4 && nt > 1) continue;   // tiny activations: occupancy matters more
    const int64_t nb = (n + 16 * nt - 1) / (16 * nt);
    // XD: wide tiles amortize each activation load over more rows; splits may
    // go down to 8 groups per workgroup
    const int64_t reach = p.xd ? nb * std::max<int64_t>(1, G / 8) : nb * ks_min;
    if (reach >= target || nt == 1) {
      p.nt = nt;
      break;
    }
  }
  // A wave's share of a k-block is bounded by the metadata it stages through
  // its registers: kMetaRounds float4 units per lane (MV).
  auto per_limit = [&](bool mv) {
    int64_t lim = G;   // a wave's share never exceeds the k range (and lim * waves cannot overflow)
    if (mv) lim = std::min<int64_t>(lim, (int64_t)kWave * kMetaRounds * 4 / (16 * p.nt));
    return lim;
  };
  p.mv = (G % 4) == 0 && gw_max >= 4 && per_limit(true) >= 4;
  const int64_t unit = p.mv ? 4 : 1;
  const int64_t per_max = std::max<int64_t>(1, per_limit(p.mv) / unit) * unit;
  const int64_t nb = (n + 16 * p.nt - 1) / (16 * p.nt);
  int64_t ks = std::max<int64_t>(ks_min, (target + nb - 1) / nb);
  ks = std::min<int64_t>(ks, std::max<int64_t>(1, G));
  // groups per k-block when wv waves share it
  auto k_block = [&](int wv) {
    const int64_t cap =
        std::max<int64_t>(unit, std::min<int64_t>(gw_max, per_max * wv) / unit * unit);
    const int64_t g = std::max<int64_t>(1, (G + ks - 1) / ks);
    return std::min<int64_t>((g + unit - 1) / unit * unit, cap);
  };
  int wv = kWaves;
  int64_t gw_wide = 0;
  if (p.mt == 1) {
    int w = p.xd ? 8 : 16;
    int64_t g = k_block(w);
    while (w > kWaves && g / unit < w) {   // at least one unit of groups per wave
      w /= 2;
      g = k_block(w);
    }
    if (w > kWaves && nb * std::max<int64_t>(1, (G + g - 1) / g) <= kWvBlocks) wv = w;
    if (wv == kWaves && p.xd) {
      // Per-lane activation loads on k-blocks too short for 8 waves with
      // 4-group metadata units: 8 waves on the same k-blocks with metadata
      // staged per group (two waves per SIMD instead of one).
      const int64_t g2 = std::max<int64_t>(1, (G + ks - 1) / ks);
      if (g2 >= 8 && g2 <= gw_max) {
        wv = 8;
        gw_wide = g2;
        p.mv = false;
      }
    }
    if (wv == kWaves && !p.xd) {
      // Small grids whose k-blocks hold too few 4-group metadata units for
      // wide workgroups: wide workgroups on fewer (or no) k splits instead,
      // with metadata staged per group (the split tails cost more than the
      // vector staging saves).
      for (int w2 : {16, 8}) {
        const int64_t ks2 = std::max<int64_t>(ks_min, (target * kWaves / w2 + nb - 1) / nb);
        const int64_t g2 = std::max<int64_t>(1, (G + ks2 - 1) / ks2);
        if (g2 > gw_max || g2 < w2 || nb * ((G + g2 - 1) / g2) > kWvBlocks) continue;
        wv = w2;
        gw_wide = g2;
        p.mv = false;
        break;
      }
    }
  }
  if (p.mt == 1 && !p.xd && m > 4) {
    // A split k on a layer narrow enough for at most kWvBlocks wide
    // workgroups: one workgroup per row tile, alone on its CU, holds the whole
    // k range's activations in the larger LDS budget, so the split (partial
    // sums and their reduction) goes away.  16-row tiles take 16 waves; wider
    // layers take 64-row tiles of 8 waves.
    const int64_t g_now = gw_wide ? gw_wide : k_block(wv);
    const int64_t gw_max_wide = (int64_t)kLdsBudgetWide / (m * 256);
    // (the activations, metadata and reduction area must fit the LDS ceiling)
    auto fits = [&](int nt, int w) { return gemv_lds_bytes(m, 1, nt, (int)G, false, w) <= kMaxDynLds; };
    if (g_now < G && G <= gw_max_wide) {
      if (G >= 16 && (n + 15) / 16 <= kWvBlocks && fits(1, 16)) {
        p.nt = 1;
        p.mv = false;
        wv = 16;
        gw_wide = G;
      } else if (G >= 8 && p.nt == 4 && (n + 63) / 64 <= kWvBlocks && fits(4, 8)) {
        // 4-group metadata vectors when every wave gets whole units within
        // its staging rounds (the 8B gate/up at M = 16: 2-7% faster than
        // per-group staging)
        const int64_t units = G / 4, per_wave = (units + 7) / 8;
        p.mv = G % 4 == 0 && units >= 8 && 4 * per_wave <= (int64_t)kWave * kMetaRounds * 4 / (16 * 4);
        wv = 8;
        gw_wide = G;
      }
    }
  }
  p.wv = wv;
  const int64_t gw = gw_wide ? gw_wide : k_block(wv);
  p.gw = (int)gw;
  p.b = (p.xd && p.mt > 1) ? 1 : p.nt == 1 ? kBatchNt1 : p.nt == 2 ? kBatchNt2 : kBatchNt4;
  p.ksplits = (int)std::max<int64_t>(1, (G + p.gw - 1) / p.gw);
  p.nblocks = (int)((n + 16 * p.nt - 1) / (16 * p.nt));
  if ((p.nblocks > kMaxTicketBlocks && p.ksplits > 1) || p.ksplits > 65535) p.ksplits = 0;   // not supported
  p.ws_bytes = p.ksplits > 1 ? kTicketBytes + (size_t)p.ksplits * m * n * sizeof(float) : 0;
  return p;
}

hipError_t launch_gemv(const uint16_t *x, const uint32_t *codes, const void *scales,
                       const uint8_t *zeros, bool compact, int64_t m, int64_t n, int64_t k,
                       int bits, float *y, void *ws, const GemvPlan &plan, hipStream_t s) {
#define SLQ_GEMV_BITS(B_)                                                                   \
  case B_:                                                                                  \
    return compact ? gemv_bits<B_, true>(x, codes, scales, zeros, m, n, k, y, ws, plan, s) \
                   : gemv_bits<B_, false>(x, codes, scales, zeros, m, n, k, y, ws, plan, s);
  switch (bits) {
    SLQ_GEMV_BITS(2)
    SLQ_GEMV_BITS(3)
    SLQ_GEMV_BITS(4)
    SLQ_GEMV_BITS(5)
    SLQ_GEMV_BITS(6)
    SLQ_GEMV_BITS(7)
    SLQ_GEMV_BITS(8)
    default: return hipErrorInvalidValue;
  }
#undef SLQ_GEMV_BITS
}

}  // namespace slq
