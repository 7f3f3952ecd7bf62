// Fidelity reductions over next-token logits for gfx950: row log-normalizer,
// EAR (sum of min(p, q)) and KL(p || q).
//
// Sources: gist.science summary "Statistically-Lossless Quantization of Large
// Language Models", Methodology 2 (EAR: summed min of the reference and
// quantized next-token distributions, averaged over positions); SLQ README,
// Evaluation (EAR and KL of a model against its base); SLQ blog, The
// Motivation (the next-token distribution is the softmax of the logits).
//
// Each row (a position) is cut into C chunks so that rows * C workgroups fill
// the chip.  Pass 1 streams a and b once per chunk and keeps, per thread, an
// online (running max, sum of exp) pair for both rows plus
//   U = sum_v exp(a_v - max_a) * (a_v - b_v),
// which gives KL without a second pass: KL = U / Z_a - (A - B), where A and B
// are the log-normalizers.  Chunk partials are combined per row in fp64 in a
// fixed order.  Pass 2 needs A and B (min(p, q) is not decomposable before
// normalization); it combines the row's chunk statistics into A, B and KL,
// sums exp(min(a - A, b - B)) = min(p, q) (one exponential per element), and
// visits rows in reverse order so the most recently streamed rows are still
// cached.  (Blocking rows so that pass 2 re-reads a block from the Infinity
// Cache measured slower at every block size.)
// Every reduction has a fixed shape, so repeated calls are bit-identical.
#include <algorithm>

#include <type_traits>

#include "launch.h"
#include "slq_device.h"

namespace slq {
namespace {

constexpr int kThreads = 256;
constexpr int64_t kRowBatch = 65535;   // rows per launch of the (chunk, row) grids: grid.y limit
constexpr double kLog2e_d = 1.4426950408889634;
constexpr float kLog2e = (float)kLog2e_d;

struct Fid {
  int C;          // chunks per row
  int64_t chunk;  // elements per chunk (multiple of 4)
};

// Chunks per row: about kFidTargetWgs workgroups per launch, chunks of at
// least 4096 elements.
#ifndef SLQ_FID_TARGET_WGS
#define SLQ_FID_TARGET_WGS 1024
#endif
constexpr int64_t kFidTargetWgs = SLQ_FID_TARGET_WGS;
Fid fid_plan(int64_t rows, int64_t vocab) {
  Fid f;
  int64_t c = (kFidTargetWgs + rows - 1) / rows;
  const int64_t maxc = std::max<int64_t>(1, (vocab + 4095) / 4096);
  c = std::min(std::max<int64_t>(c, 1), maxc);
  int64_t chunk = (vocab + c - 1) / c;
  chunk = (chunk + 3) & ~(int64_t)3;
  f.C = (int)((vocab + chunk - 1) / chunk);
  f.chunk = chunk;
  return f;
}

// Workspace (8-byte words): stats [rows][C][5] | rowres [rows][4] |
// earpart [rows][C] | top-K keys u64 [rows][C][kTopKMax] |
// top-K quantized logits f32 [rows][C][kTopKMax] (half a word each) | pad |
// top-K ticket u32
size_t ws_doubles(int64_t rows, const Fid &f) {
  return (size_t)rows * f.C * 5 + (size_t)rows * 4 + (size_t)rows * f.C +
         (size_t)rows * f.C * kTopKMax + (size_t)rows * f.C * kTopKMax / 2 + 2;
}

// The hardware base-2 exponential (v_exp_f32).  Arguments here are
// (logit - running max) * log2(e) / T <= 0, so only terms below 2^-126 of the
// running maximum flush to zero: negligible next to a sum that is >= 1 and
// the 1e-5 tolerance of EAR and KL.  exp2f adds a denormal-range fix-up of
// about five instructions per call around the same instruction, which made
// the first pass VALU-bound.
__device__ __forceinline__ float exp2_hw(float v) { return __builtin_amdgcn_exp2f(v); }
__device__ __forceinline__ float fast_exp(float v) { return exp2_hw(v * kLog2e); }

// (m, z, u) combine: z, u are sums of exp(. - m).
struct MZ {
  double m, z, u;
};
// invT: the sums are of exp((x - m) * invT) (a softmax at temperature 1 / invT).
__device__ __forceinline__ MZ mz_combine(MZ p, MZ q, double invT = 1.0) {
  if (q.m == -INFINITY) return p;
  if (p.m == -INFINITY) return q;
  const double M = p.m > q.m ? p.m : q.m;
  const double fp = exp((p.m - M) * invT), fq = exp((q.m - M) * invT);
  return MZ{M, p.z * fp + q.z * fq, p.u * fp + q.u * fq};
}
__device__ __forceinline__ MZ mz_shfl(MZ v, int o) {
  return MZ{__shfl_xor(v.m, o, kWave), __shfl_xor(v.z, o, kWave), __shfl_xor(v.u, o, kWave)};
}
__device__ MZ mz_block(MZ v, MZ *lds, double invT) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) v = mz_combine(v, mz_shfl(v, o), invT);
  const int wave = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) lds[wave] = v;
  __syncthreads();
  MZ t = lds[0];
  for (int i = 1; i < kThreads / kWave; ++i) t = mz_combine(t, lds[i], invT);
  return t;
}

// Online update of (m, z, u) with 4 new values of a (u only when WITH_U); the
// terms are exp2((a - m) * c) with c = log2(e) / temperature.  The shift by the
// running maximum comes before the scaling, so large logits lose nothing to it.
// The difference a - b enters u in fp64, where it is exact: with logits far
// from zero an fp32 difference would lose more than the KL being measured.
template <bool WITH_U>
__device__ __forceinline__ void online4(float4 a, float4 b, float &m, double &z, double &u,
                                        float c) {
  const float mx = fmaxf(fmaxf(a.x, a.y), fmaxf(a.z, a.w));
  if (mx > m) {
    const float f = exp2_hw((m - mx) * c);   // m = -inf gives 0
    z *= (double)f;
    if (WITH_U) u *= (double)f;
    m = mx;
  }
  const float e0 = exp2_hw((a.x - m) * c), e1 = exp2_hw((a.y - m) * c), e2 = exp2_hw((a.z - m) * c),
              e3 = exp2_hw((a.w - m) * c);
  if (!WITH_U) {
    z += (double)((e0 + e1) + (e2 + e3));
  } else {
    // U / Z is a p-weighted mean of a - b, which can be large next to the KL:
    // both sums take exactly the same fp64 weights.
    z += (double)e0;
    z += (double)e1;
    z += (double)e2;
    z += (double)e3;
    u = fma((double)e0, (double)a.x - (double)b.x, u);
    u = fma((double)e1, (double)a.y - (double)b.y, u);
    u = fma((double)e2, (double)a.z - (double)b.z, u);
    u = fma((double)e3, (double)a.w - (double)b.w, u);
  }
}

// Online update with one value (rows whose length is not a multiple of 4).
template <bool WITH_U>
__device__ __forceinline__ void online1(float a, float b, float &m, double &z, double &u,
                                        float c) {
  if (a > m) {
    const float f = exp2_hw((m - a) * c);
    z *= (double)f;
    if (WITH_U) u *= (double)f;
    m = a;
  }
  const float e = exp2_hw((a - m) * c);
  z += (double)e;
  if (WITH_U) u = fma((double)e, (double)a - (double)b, u);
}

// Pass 1: per (chunk, row) partial (m_a, Z_a, U, m_b, Z_b).
// At temperature T: escale = log2(e) / T and invT = 1 / T (log2(e) and 1 for
// the plain metrics); m stays in the logits' own units.
template <bool WITH_B>
__global__ __launch_bounds__(kThreads) void stats_kernel(const float *__restrict__ a,
                                                         const float *__restrict__ b,
                                                         int64_t vocab, Fid f, int64_t r0,
                                                         float escale, double invT,
                                                         double *__restrict__ stats) {
  __shared__ MZ lds[kThreads / kWave];
  const int c = blockIdx.x;
  const int64_t row = r0 + blockIdx.y;
  const int64_t beg = (int64_t)c * f.chunk;
  const int64_t end = std::min<int64_t>(beg + f.chunk, vocab);
  const float *ar = a + row * vocab;
  const float *br = WITH_B ? b + row * vocab : nullptr;

  float ma = -INFINITY, mb = -INFINITY;
  double za = 0.0, ua = 0.0, zb = 0.0, ub = 0.0;
  const bool vec = ((vocab & 3) == 0);
  if (vec) {
    const float4 *a4 = reinterpret_cast<const float4 *>(ar);
    const float4 *b4 = WITH_B ? reinterpret_cast<const float4 *>(br) : nullptr;
    for (int64_t i = beg / 4 + threadIdx.x; i < end / 4; i += kThreads) {
      const float4 va = a4[i];
      if (WITH_B) {
        const float4 vb = b4[i];
        online4<true>(va, vb, ma, za, ua, escale);
        online4<false>(vb, vb, mb, zb, ub, escale);
      } else {
        online4<false>(va, va, ma, za, ua, escale);
      }
    }
  } else {
    for (int64_t i = beg + threadIdx.x; i < end; i += kThreads) {
      const float va = ar[i];
      const float vb = WITH_B ? br[i] : 0.f;
      online1<WITH_B>(va, vb, ma, za, ua, escale);
      if (WITH_B) online1<false>(vb, vb, mb, zb, ub, escale);
    }
  }
  const MZ ra = mz_block(MZ{(double)ma, za, ua}, lds, invT);
  MZ rb{0.0, 0.0, 0.0};
  if (WITH_B) rb = mz_block(MZ{(double)mb, zb, 0.0}, lds, invT);
  if (threadIdx.x == 0) {
    double *o = stats + (row * f.C + c) * 5;
    o[0] = ra.m;
    o[1] = ra.z;
    o[2] = ra.u;
    o[3] = rb.m;
    o[4] = rb.z;
  }
}

// Per row: combine chunk partials in chunk order -> A, B, KL.
template <bool WITH_B>
__global__ __launch_bounds__(kThreads) void rows_kernel(const double *__restrict__ stats, int64_t r0,
                                                        int64_t r1, Fid f, double *__restrict__ rowres,
                                                        double *__restrict__ lse_out,
                                                        float *__restrict__ kl_rows) {
  const int64_t r = r0 + (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (r >= r1) return;
  MZ ta{-INFINITY, 0.0, 0.0}, tb{-INFINITY, 0.0, 0.0};
  for (int c = 0; c < f.C; ++c) {
    const double *s = stats + (r * f.C + c) * 5;
    ta = mz_combine(ta, MZ{s[0], s[1], s[2]});
    if (WITH_B) tb = mz_combine(tb, MZ{s[3], s[4], 0.0});
  }
  const double A = ta.m + log(ta.z);
  if (!WITH_B) {
    lse_out[r] = A;
    return;
  }
  const double B = tb.m + log(tb.z);
  const double kl = ta.u / ta.z - (A - B);
  rowres[r * 4 + 0] = A;
  rowres[r * 4 + 1] = B;
  rowres[r * 4 + 2] = kl;
  kl_rows[r] = (float)kl;
}

__device__ __forceinline__ double block_sum_f64(double v, double *lds) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) v += __shfl_xor(v, o, kWave);
  const int wave = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) lds[wave] = v;
  __syncthreads();
  double t = 0.0;
  for (int i = 0; i < kThreads / kWave; ++i) t += lds[i];
  return t;
}

// Pass 2: per (chunk, row) partial of sum min(exp(a - A), exp(b - B)).
// Pass 2 also combines the row's chunk statistics (in chunk order, the same
// arithmetic in every workgroup of the row) into A, B and KL; chunk 0 records
// them for the final means.
__global__ __launch_bounds__(kThreads) void ear_kernel(const float *__restrict__ a,
                                                       const float *__restrict__ b, int64_t row_end,
                                                       int64_t vocab, Fid f,
                                                       const double *__restrict__ stats,
                                                       double *__restrict__ rowres,
                                                       float *__restrict__ kl_rows,
                                                       double *__restrict__ earpart) {
  __shared__ double lds[kThreads / kWave];
  __shared__ double ab[2];
  const int c = blockIdx.x;
  // rows below row_end in reverse order of pass 1: the most recent rows are still cached
  const int64_t row = row_end - 1 - blockIdx.y;
  if (threadIdx.x == 0) {
    MZ ta{-INFINITY, 0.0, 0.0}, tb{-INFINITY, 0.0, 0.0};
    for (int cc = 0; cc < f.C; ++cc) {
      const double *st = stats + (row * f.C + cc) * 5;
      ta = mz_combine(ta, MZ{st[0], st[1], st[2]});
      tb = mz_combine(tb, MZ{st[3], st[4], 0.0});
    }
    const double A = ta.m + log(ta.z), B = tb.m + log(tb.z);
    ab[0] = A;
    ab[1] = B;
    if (c == 0) {
      const double kl = ta.u / ta.z - (A - B);
      rowres[row * 4 + 0] = A;
      rowres[row * 4 + 1] = B;
      rowres[row * 4 + 2] = kl;
      kl_rows[row] = (float)kl;
    }
  }
  __syncthreads();
  const int64_t beg = (int64_t)c * f.chunk;
  const int64_t end = std::min<int64_t>(beg + f.chunk, vocab);
  // a - A is formed as (a - A_hi) - A_lo with A = A_hi + A_lo split into two
  // floats: the first subtraction is exact wherever p is not negligible, so
  // the exponent keeps full fp32 accuracy even for logits far from zero.
  const double Ad = ab[0], Bd = ab[1];
  const float Ahi = (float)Ad, Alo = (float)(Ad - (double)Ahi);
  const float Bhi = (float)Bd, Blo = (float)(Bd - (double)Bhi);
  const float *ar = a + row * vocab;
  const float *br = b + row * vocab;
  double acc = 0.0;
  if ((vocab & 3) == 0) {
    const float4 *a4 = reinterpret_cast<const float4 *>(ar);
    const float4 *b4 = reinterpret_cast<const float4 *>(br);
    for (int64_t i = beg / 4 + threadIdx.x; i < end / 4; i += kThreads) {
      const float4 va = a4[i], vb = b4[i];
      // min(e^x, e^y) = e^min(x, y): one exponential per element
      const float m0 = fast_exp(fminf((va.x - Ahi) - Alo, (vb.x - Bhi) - Blo));
      const float m1 = fast_exp(fminf((va.y - Ahi) - Alo, (vb.y - Bhi) - Blo));
      const float m2 = fast_exp(fminf((va.z - Ahi) - Alo, (vb.z - Bhi) - Blo));
      const float m3 = fast_exp(fminf((va.w - Ahi) - Alo, (vb.w - Bhi) - Blo));
      acc += (double)((m0 + m1) + (m2 + m3));
    }
  } else {
    for (int64_t i = beg + threadIdx.x; i < end; i += kThreads) {
      acc += (double)fast_exp(fminf((ar[i] - Ahi) - Alo, (br[i] - Bhi) - Blo));
    }
  }
  const double t = block_sum_f64(acc, lds);
  if (threadIdx.x == 0) earpart[row * f.C + c] = t;
}

// Per row EAR, then the two means; one workgroup, fixed order.
__global__ __launch_bounds__(kThreads) void final_kernel(const double *__restrict__ earpart,
                                                         const double *__restrict__ rowres,
                                                         int64_t rows, Fid f,
                                                         float *__restrict__ ear_rows,
                                                         double *__restrict__ means) {
  __shared__ double lds[kThreads / kWave];
  double se = 0.0, sk = 0.0;
  for (int64_t r = threadIdx.x; r < rows; r += kThreads) {
    double e = 0.0;
    for (int c = 0; c < f.C; ++c) e += earpart[r * f.C + c];
    ear_rows[r] = (float)e;
    se += e;
    sk += rowres[r * 4 + 2];
  }
  const double te = block_sum_f64(se, lds);
  const double tk = block_sum_f64(sk, lds);
  if (threadIdx.x == 0) {
    means[0] = rows > 0 ? te / (double)rows : 0.0;
    means[1] = rows > 0 ? tk / (double)rows : 0.0;
  }
}

// ---- top-K EAR / top-K KL ----
// A token's selection key: larger logit first, then lower index.  Float bits
// are mapped to an order-preserving unsigned integer in the high half; the
// complemented index fills the low half, so keys of one row are distinct and
// every real key is above 0.
__device__ __forceinline__ uint64_t topk_key(float v, uint32_t idx) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)o << 32) | (uint64_t)(0xFFFFFFFFu - idx);
}
__device__ __forceinline__ float topk_value(uint64_t key) {
  const uint32_t o = (uint32_t)(key >> 32);
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

constexpr int kCandCap = 512;   // per-wave candidate buffer (entries)

// The K-th largest of the keys the wave holds (PER per lane, 0 = no entry),
// by radix selection from the top bit down: a bit is kept when at least K keys
// lie at or above the prefix with it set.  Counts are popcounts of ballots, so
// the search runs in scalar registers with no data exchange between lanes.
// Keys are distinct, so exactly K keys are >= the result; the low half is only
// searched when the high half leaves a tie.  Needs >= K nonzero keys.
template <int PER>
__device__ uint64_t kth_key(const uint64_t (&key)[PER], int k) {
  uint64_t prefix = 0;
  for (int bit = 63; bit >= 0; --bit) {
    const uint64_t cand = prefix | (1ull << bit);
    int cnt = 0;
#pragma unroll
    for (int r = 0; r < PER; ++r) cnt += __popcll(__ballot(key[r] >= cand));
    if (cnt >= k) prefix = cand;
    if (bit == 32) {
      int at = 0;
#pragma unroll
      for (int r = 0; r < PER; ++r) at += __popcll(__ballot(key[r] >= prefix));
      if (at == k) return prefix;
    }
  }
  return prefix;
}

// wave_keep with the buffer's first `count` entries in PER registers per lane.
template <int PER>
__device__ int keep_in_regs(uint64_t *ck, float *cb, int count, int k, uint64_t &kth) {
  const int lane = threadIdx.x & (kWave - 1);
  const uint64_t below = (1ull << lane) - 1;
  uint64_t key[PER];
  float bv[PER];
#pragma unroll
  for (int r = 0; r < PER; ++r) {
    const int e = r * kWave + lane;
    key[r] = e < count ? ck[e] : 0;
    bv[r] = e < count ? cb[e] : 0.f;
  }
  kth = kth_key<PER>(key, k);
  int base = 0;
#pragma unroll
  for (int r = 0; r < PER; ++r) {
    const bool keep = key[r] >= kth;
    const uint64_t m = __ballot(keep);
    if (keep) {
      const int pos = base + __popcll(m & below);
      ck[pos] = key[r];
      cb[pos] = bv[r];
    }
    base += __popcll(m);
  }
  return k;
}

// Cuts one wave's candidate buffer (first `count` entries) back to its k
// largest keys, stored at the front in lane order.  Returns the new count;
// `kth` is the smallest key kept when the buffer held more than k, else 0.
template <int CAP>
__device__ int wave_keep(uint64_t *ck, float *cb, int count, int k, uint64_t &kth) {
  kth = 0;
  if (count <= k) return count;
  // as few registers per lane as hold the entries: the selection costs one
  // ballot per register and key bit
  if (count <= kWave) return keep_in_regs<1>(ck, cb, count, k, kth);
  if constexpr (CAP >= 2 * kWave)
    if (count <= 2 * kWave) return keep_in_regs<2>(ck, cb, count, k, kth);
  if constexpr (CAP >= 4 * kWave)
    if (count <= 4 * kWave) return keep_in_regs<4>(ck, cb, count, k, kth);
  return keep_in_regs<CAP / kWave>(ck, cb, count, k, kth);
}

// Pass 1 of the top-K metrics, per (chunk, row): the chunk's softmax partials
// (m, Z) of both logit rows at temperature T, and the chunk's K largest
// reference keys with the quantized model's logit at each (in no particular
// order; key 0 pads a chunk shorter than K).  Each wave filters its elements
// against a rising threshold (the K-th largest value it has kept) into an LDS
// buffer and cuts the buffer back to K whenever it could overflow; the four
// waves' lists are merged at the end.  Also clears pass 2's ticket.
template <int KT>
__global__ __launch_bounds__(kThreads) void topk_stats_kernel(
    const float *__restrict__ a, const float *__restrict__ b, int64_t vocab, Fid f, int64_t r0,
    int k, float escale, double invT, double *__restrict__ stats, uint64_t *__restrict__ cand_key,
    float *__restrict__ cand_b, unsigned *__restrict__ ticket) {
  __shared__ MZ lds[kThreads / kWave];
  __shared__ uint64_t ck[kThreads / kWave][kCandCap];
  __shared__ float cb[kThreads / kWave][kCandCap];
  const int c = blockIdx.x;
  const int64_t row = r0 + blockIdx.y;
  const int64_t beg = (int64_t)c * f.chunk;
  const int64_t end = std::min<int64_t>(beg + f.chunk, vocab);
  const float *ar = a + row * vocab;
  const float *br = b + row * vocab;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  uint64_t *wk = ck[wave];
  float *wb = cb[wave];

  float ma = -INFINITY, mb = -INFINITY;
  double za = 0.0, zb = 0.0, unused = 0.0;
  int n = 0;                  // wave-uniform buffer fill
  float theta = -INFINITY;    // wave-uniform admission threshold
  const uint64_t below = (1ull << lane) - 1;
  auto offer = [&](bool ok, float v, float bvv, uint32_t idx) {
    const bool in = ok && v >= theta;
    const uint64_t mask = __ballot(in);
    if (mask) {
      if (in) {
        const int pos = n + __popcll(mask & below);
        wk[pos] = topk_key(v, idx);
        wb[pos] = bvv;
      }
      n += __popcll(mask);
    }
  };
  auto compact = [&]() {
    if (n > kCandCap - 4 * kWave) {   // the next offers could overflow: n > 256 >= k
      uint64_t kth;
      n = wave_keep<kCandCap>(wk, wb, n, k, kth);
      theta = topk_value(kth);
    }
  };
  if ((vocab & 3) == 0) {
    const float4 *a4 = reinterpret_cast<const float4 *>(ar);
    const float4 *b4 = reinterpret_cast<const float4 *>(br);
    constexpr int kU = 4;   // float4 pairs in flight per lane
    // same trip count for all lanes of the wave (the ballots need every lane)
    for (int64_t i0 = beg / 4; i0 < end / 4; i0 += kU * kThreads) {
      float4 va[kU], vb[kU];
      bool ok[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int64_t i = i0 + u * kThreads + threadIdx.x;
        ok[u] = i < end / 4;
        va[u] = vb[u] = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
        if (ok[u]) {
          va[u] = a4[i];
          vb[u] = b4[i];
        }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int u = 0; u < kU; ++u)
        if (ok[u]) {
          online4<false>(va[u], va[u], ma, za, unused, escale);
          online4<false>(vb[u], vb[u], mb, zb, unused, escale);
          mx = fmaxf(mx, fmaxf(fmaxf(va[u].x, va[u].y), fmaxf(va[u].z, va[u].w)));
        }
      if (theta == -INFINITY) {
        // First batch: the K-th largest of the lanes' maxima (K distinct
        // elements) bounds the wave's K-th largest value from below, so it can
        // serve as the threshold before any offer; lanes without elements
        // take key 0, which ranks below every element.
        uint64_t lk[1] = {mx > -INFINITY ? topk_key(mx, (uint32_t)lane) : 0ull};
        if (__popcll(__ballot(lk[0] != 0ull)) >= k) theta = topk_value(kth_key<1>(lk, k));
      }
      if (__ballot(mx >= theta)) {   // rare once the threshold has risen
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const uint32_t base = (uint32_t)(4 * (i0 + u * kThreads + threadIdx.x));
          offer(ok[u], va[u].x, vb[u].x, base);
          offer(ok[u], va[u].y, vb[u].y, base + 1);
          offer(ok[u], va[u].z, vb[u].z, base + 2);
          offer(ok[u], va[u].w, vb[u].w, base + 3);
          compact();
        }
      }
    }
  } else {
    for (int64_t i0 = beg; i0 < end; i0 += kThreads) {
      const int64_t i = i0 + threadIdx.x;
      const bool ok = i < end;
      float va = -INFINITY, vb = -INFINITY;
      if (ok) {
        va = ar[i];
        vb = br[i];
        online1<false>(va, va, ma, za, unused, escale);
        online1<false>(vb, vb, mb, zb, unused, escale);
      }
      offer(ok, va, vb, (uint32_t)i);
      compact();
    }
  }
  const MZ ra = mz_block(MZ{(double)ma, za, 0.0}, lds, invT);
  const MZ rb = mz_block(MZ{(double)mb, zb, 0.0}, lds, invT);
  // each wave's top min(n, k), then wave 0 merges the four lists
  __shared__ uint64_t mk[kThreads / kWave * KT];
  __shared__ float mbv[kThreads / kWave * KT];
  __shared__ int mcount[kThreads / kWave];
  uint64_t kth;
  const int take = wave_keep<kCandCap>(wk, wb, n, k, kth);
  for (int j = lane; j < KT; j += kWave) {
    mk[wave * KT + j] = j < take ? wk[j] : 0;
    mbv[wave * KT + j] = j < take ? wb[j] : 0.f;
  }
  if (lane == 0) mcount[wave] = take;
  if (r0 == 0 && c == 0 && blockIdx.y == 0 && threadIdx.x == 0) *ticket = 0u;   // for pass 2
  __syncthreads();
  if (wave == 0) {
    constexpr int PER = kThreads / kWave * KT / kWave;
    int total = 0;
#pragma unroll
    for (int w = 0; w < kThreads / kWave; ++w) total += mcount[w];
    uint64_t key[PER];
    float bv[PER];
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      key[r] = mk[r * kWave + lane];
      bv[r] = mbv[r * kWave + lane];
    }
    const uint64_t thr = total > k ? kth_key<PER>(key, k) : 1;   // every real key is >= 1
    uint64_t *ok_ = cand_key + (row * f.C + c) * kTopKMax;
    float *ob = cand_b + (row * f.C + c) * kTopKMax;
    const uint64_t below = (1ull << lane) - 1;
    int base = 0;
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      const bool keep = key[r] >= thr;
      const uint64_t m = __ballot(keep);
      if (keep) {
        const int pos = base + __popcll(m & below);
        ok_[pos] = key[r];
        ob[pos] = bv[r];
      }
      base += __popcll(m);
    }
    for (int j = base + lane; j < k; j += kWave) {   // fewer than k elements in the chunk
      ok_[j] = 0;
      ob[j] = 0.f;
    }
    if (lane == 0) {
      double *o = stats + (row * f.C + c) * 5;
      o[0] = ra.m;
      o[1] = ra.z;
      o[2] = 0.0;
      o[3] = rb.m;
      o[4] = rb.z;
    }
  }
}

// Pass 2, one wave per row: the row's normalizers from the chunk partials, the
// K-th largest key among the chunk lists by radix selection, and the EAR and
// KL terms of the K keys at or above it in fp64 (lane order, then a fixed
// tree).  The last workgroup to finish (ticket) forms the means over all rows
// in a fixed order.
__global__ __launch_bounds__(kThreads) void topk_rows_kernel(
    const double *__restrict__ stats, const uint64_t *__restrict__ cand_key,
    const float *__restrict__ cand_b, int64_t rows, Fid f, int k, double invT,
    double *__restrict__ rowres, float *__restrict__ ear_rows, float *__restrict__ kl_rows,
    unsigned *__restrict__ ticket, double *__restrict__ means) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int64_t row = (int64_t)blockIdx.x * (kThreads / kWave) + wave;
  if (row < rows) {
    double st[4] = {0.0, 0.0, 0.0, 0.0};   // m_a, log Z_a, m_b, log Z_b
    if (lane == 0) {
      MZ ta{-INFINITY, 0.0, 0.0}, tb{-INFINITY, 0.0, 0.0};
      for (int c = 0; c < f.C; ++c) {
        const double *sp = stats + (row * f.C + c) * 5;
        ta = mz_combine(ta, MZ{sp[0], sp[1], 0.0}, invT);
        tb = mz_combine(tb, MZ{sp[3], sp[4], 0.0}, invT);
      }
      st[0] = ta.m;
      st[1] = log(ta.z);
      st[2] = tb.m;
      st[3] = log(tb.z);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) st[i] = __shfl(st[i], 0, kWave);
    const int64_t ne = (int64_t)f.C * k;   // chunk c's list: entries [c * kTopKMax, + k)
    const uint64_t *rk = cand_key + row * f.C * kTopKMax;
    const float *rb = cand_b + row * f.C * kTopKMax;
    auto at = [&](int64_t e) { return (e / k) * kTopKMax + e % k; };
    auto term = [&](uint64_t key, float bq, double &e, double &d) {
      const double lp = ((double)topk_value(key) - st[0]) * invT - st[1];
      const double lq = ((double)bq - st[2]) * invT - st[3];
      const double p = exp(lp), q = exp(lq);
      e += p < q ? p : q;
      d += p * (lp - lq);
    };
    double e = 0.0, d = 0.0;
    // lists of up to 1024 entries stay in registers, as few per lane as fit
    // (the selection costs one ballot per register and key bit)
    auto in_regs = [&](auto per_tag) {
      constexpr int kPer = decltype(per_tag)::value;
      uint64_t key[kPer];
#pragma unroll
      for (int r = 0; r < kPer; ++r) {
        const int64_t i = (int64_t)r * kWave + lane;
        key[r] = i < ne ? rk[at(i)] : 0;
      }
      const uint64_t thr = kth_key<kPer>(key, k);
#pragma unroll
      for (int r = 0; r < kPer; ++r)
        if (key[r] >= thr) term(key[r], rb[at((int64_t)r * kWave + lane)], e, d);
    };
    if (ne <= kWave) {
      in_regs(std::integral_constant<int, 1>{});
    } else if (ne <= 2 * kWave) {
      in_regs(std::integral_constant<int, 2>{});
    } else if (ne <= 4 * kWave) {
      in_regs(std::integral_constant<int, 4>{});
    } else if (ne <= 8 * kWave) {
      in_regs(std::integral_constant<int, 8>{});
    } else if (ne <= 16 * kWave) {
      in_regs(std::integral_constant<int, 16>{});
    } else {   // long lists (few rows, long vocabulary): count from memory
      uint64_t prefix = 0;
      for (int bit = 63; bit >= 0; --bit) {
        const uint64_t cand = prefix | (1ull << bit);
        int cnt = 0;
        for (int64_t i0 = 0; i0 < ne; i0 += kWave) {
          const int64_t i = i0 + lane;
          cnt += __popcll(__ballot(i < ne && rk[at(i < ne ? i : 0)] >= cand));
        }
        if (cnt >= k) prefix = cand;
      }
      for (int64_t i = lane; i < ne; i += kWave) {
        const uint64_t key = rk[at(i)];
        if (key >= prefix) term(key, rb[at(i)], e, d);
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {   // fixed-shape tree sum over the wave
      e += __shfl_xor(e, o, kWave);
      d += __shfl_xor(d, o, kWave);
    }
    if (lane == 0) {
      // device-scope stores: coherent across XCDs without an L2 writeback
      // (a device-scope fence here wrote back the L2 once per wave)
      __hip_atomic_store(&rowres[row * 4 + 2], d, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&rowres[row * 4 + 3], e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      ear_rows[row] = (float)e;
      kl_rows[row] = (float)d;
    }
  }
  __shared__ bool last;
  __shared__ double lds[kThreads / kWave];
  // every row result of this workgroup has completed before its ticket
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0)
    last = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
           gridDim.x - 1;
  __syncthreads();
  if (!last) return;
  double se = 0.0, sk = 0.0;
  for (int64_t r = threadIdx.x; r < rows; r += kThreads) {
    se += __hip_atomic_load(&rowres[r * 4 + 3], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sk += __hip_atomic_load(&rowres[r * 4 + 2], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  const double te = block_sum_f64(se, lds);
  const double tk = block_sum_f64(sk, lds);
  if (threadIdx.x == 0) {
    means[0] = te / (double)rows;
    means[1] = tk / (double)rows;
  }
}

}  // namespace

size_t fidelity_workspace(int64_t rows, int64_t vocab) {
  if (rows <= 0 || vocab <= 0) return 0;
  return ws_doubles(rows, fid_plan(rows, vocab)) * sizeof(double);
}

hipError_t launch_row_lse(const float *a, int64_t rows, int64_t vocab, double *lse, void *ws,
                          hipStream_t s) {
  const Fid f = fid_plan(rows, vocab);
  double *stats = static_cast<double *>(ws);
  hipError_t e;
  for (int64_t r0 = 0; r0 < rows; r0 += kRowBatch) {
    const unsigned nr = (unsigned)std::min<int64_t>(kRowBatch, rows - r0);
    hipLaunchKernelGGL((stats_kernel<false>), dim3(f.C, nr), dim3(kThreads), 0, s, a, nullptr,
                       vocab, f, r0, kLog2e, 1.0, stats);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL((rows_kernel<false>), dim3((unsigned)((rows + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, s, stats, (int64_t)0, rows, f, nullptr, lse, nullptr);
  return hipGetLastError();
}

hipError_t launch_ear_kl(const float *a, const float *b, int64_t rows, int64_t vocab, float *ear,
                         float *kl, double *means, void *ws, hipStream_t s) {
  const Fid f = fid_plan(rows, vocab);
  double *stats = static_cast<double *>(ws);
  double *rowres = stats + (size_t)rows * f.C * 5;
  double *earpart = rowres + (size_t)rows * 4;
  hipError_t e;
  for (int64_t r0 = 0; r0 < rows; r0 += kRowBatch) {
    const unsigned nr = (unsigned)std::min<int64_t>(kRowBatch, rows - r0);
    hipLaunchKernelGGL((stats_kernel<true>), dim3(f.C, nr), dim3(kThreads), 0, s, a, b, vocab, f,
                       r0, kLog2e, 1.0, stats);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  for (int64_t hi = rows; hi > 0; hi -= kRowBatch) {   // last rows first, as they were read last
    const unsigned nr = (unsigned)std::min<int64_t>(kRowBatch, hi);
    hipLaunchKernelGGL(ear_kernel, dim3(f.C, nr), dim3(kThreads), 0, s, a, b, hi, vocab, f, stats,
                       rowres, kl, earpart);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(final_kernel, dim3(1), dim3(kThreads), 0, s, earpart, rowres, rows, f, ear,
                     means);
  return hipGetLastError();
}

hipError_t launch_ear_kl_topk(const float *a, const float *b, int64_t rows, int64_t vocab, int k,
                              double invT, float *ear, float *kl, double *means, void *ws,
                              hipStream_t s) {
  const Fid f = fid_plan(rows, vocab);
  double *stats = static_cast<double *>(ws);
  double *rowres = stats + (size_t)rows * f.C * 5;
  uint64_t *cand_key = reinterpret_cast<uint64_t *>(rowres + (size_t)rows * 4 + (size_t)rows * f.C);
  float *cand_b = reinterpret_cast<float *>(cand_key + (size_t)rows * f.C * kTopKMax);
  unsigned *ticket = reinterpret_cast<unsigned *>(cand_b + (size_t)rows * f.C * kTopKMax + 1);
  const float escale = (float)(kLog2e_d * invT);
  hipError_t e;
  for (int64_t r0 = 0; r0 < rows; r0 += kRowBatch) {
    const dim3 grid(f.C, (unsigned)std::min<int64_t>(kRowBatch, rows - r0));
    if (k <= 16)
      hipLaunchKernelGGL((topk_stats_kernel<16>), grid, dim3(kThreads), 0, s, a, b, vocab, f, r0,
                         k, escale, invT, stats, cand_key, cand_b, ticket);
    else if (k <= 32)
      hipLaunchKernelGGL((topk_stats_kernel<32>), grid, dim3(kThreads), 0, s, a, b, vocab, f, r0,
                         k, escale, invT, stats, cand_key, cand_b, ticket);
    else
      hipLaunchKernelGGL((topk_stats_kernel<kTopKMax>), grid, dim3(kThreads), 0, s, a, b, vocab, f,
                         r0, k, escale, invT, stats, cand_key, cand_b, ticket);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const unsigned wgs = (unsigned)((rows + kThreads / kWave - 1) / (kThreads / kWave));
  hipLaunchKernelGGL(topk_rows_kernel, dim3(wgs), dim3(kThreads), 0, s, stats, cand_key, cand_b,
                     rows, f, k, invT, rowres, ear, kl, ticket, means);
  return hipGetLastError();
}

}  // namespace slq
