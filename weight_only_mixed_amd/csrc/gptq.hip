// GPTQ code selection for gfx950 (named by the SLQ README, Pipeline, as the
// code-choice step: layer-wise GPTQ at every bit-width, asymmetric INT, group
// size 128; the steps follow the published algorithm: Frantar et al., "GPTQ:
// Accurate Post-Training Quantization for Generative Pre-trained
// Transformers", Algorithm 1 with the Cholesky form of the inverse Hessian and
// lazy batched updates).
//
//  1. Dead inputs (H_ii = 0) get H_ii = 1 and a zeroed weight column; then
//     H += damp * mean(diag H) * I.
//  2. The upper factor U with U^T U = H^-1: with J the index reversal and
//     J H J = L L^T (lower Cholesky factor), H^-1 = (J L^-1 J)^T (J L^-1 J), so
//     U = J L^-1 J.  The reversed matrix is factored in fp64 by a blocked
//     right-looking Cholesky (64 x 64 diagonal blocks in LDS, a panel solve and
//     a tiled trailing update), and L is inverted by right-looking block
//     substitution (every step a grid of tile updates).
//  3. Columns in groups of 128 (the lazy batch is the group), in fp32 with
//     one rounding per operation (built without contraction): per weight row,
//     a team of lanes holds the group's 128 current weights, computes the
//     group's scale and zero point from them (the plain quantizer's steps),
//     and for each column i quantizes it, takes e_i = (w_i - w_hat_i) / U_ii
//     and moves the group's later columns by w_j = fma(-e_i, U_ij, w_j).  A
//     tiled update then moves every later column c of the layer once:
//     w_c -= a_c, a_c the fma chain of e_p * U[i1 + p][c] over p = 0..127.
//  Steps 1-2 (the factor) and 3 (the column pass) are separate entry points
//  as well, so one factor serves the layer at every bit-width.
#include <cmath>

#include "launch.h"
#include "slq_device.h"

namespace slq {
namespace {

constexpr int kThr = 256;
constexpr int kNb = 64;   // Cholesky / inverse block
constexpr int kLdp = kNb + 1;

__device__ __forceinline__ double block_sum(double v, double *lds) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) lds[w] = v;
  __syncthreads();
  double t = 0.0;
  for (int i = 0; i < kThr / kWave; ++i) t += lds[i];
  return t;
}

// mean of the diagonal after dead inputs get 1 (one workgroup, fixed order),
// and the dead-input mask (H_ii == 0: the input never fires)
__global__ __launch_bounds__(kThr) void diag_mean_kernel(const float *__restrict__ H, int64_t k,
                                                         double *__restrict__ stat,
                                                         uint8_t *__restrict__ dead) {
  __shared__ double lds[kThr / kWave];
  double s = 0.0;
  for (int64_t i = threadIdx.x; i < k; i += kThr) {
    const float h = H[i * k + i];
    s += h == 0.0f ? 1.0 : (double)h;
    dead[i] = h == 0.0f ? 1 : 0;
  }
  const double t = block_sum(s, lds);
  if (threadIdx.x == 0) stat[0] = t / (double)k;
}

// A = J H' J in fp64 (H' = H with dead diagonals 1 and the damping added)
__global__ __launch_bounds__(kThr) void prep_kernel(const float *__restrict__ H, int64_t k,
                                                    double damp, const double *__restrict__ stat,
                                                    double *__restrict__ A) {
  const int64_t e = (int64_t)blockIdx.x * kThr + threadIdx.x;
  if (e >= k * k) return;
  const int64_t i = e / k, j = e % k;
  const int64_t si = k - 1 - i, sj = k - 1 - j;
  double h = (double)H[si * k + sj];
  if (si == sj) {
    if (h == 0.0) h = 1.0;
    h += damp * stat[0];
  }
  A[e] = h;
}

// working weights: dead input columns zeroed (no mask: none is dead)
__global__ __launch_bounds__(kThr) void wcopy_kernel(const float *__restrict__ W,
                                                     const uint8_t *__restrict__ dead, int64_t n,
                                                     int64_t k, float *__restrict__ Wk) {
  const int64_t e = (int64_t)blockIdx.x * kThr + threadIdx.x;
  if (e >= n * k) return;
  const int64_t c = e % k;
  Wk[e] = dead && dead[c] ? 0.0f : W[e];
}

// Cholesky of the diagonal block at j0: one wavefront, lane i holds row i of
// the block in registers.  Column c: the pivot and then each scaled entry of
// column c are broadcast from their lanes (readlane), and every lane updates
// its own row.  Entries right of a lane's diagonal receive junk and are never
// stored.
__device__ __forceinline__ double lane_bcast(double v, int lane) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)b, lane);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(b >> 32), lane);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

__global__ __launch_bounds__(kNb) void potf2_kernel(double *__restrict__ A, int64_t k, int64_t j0) {
  const int i = threadIdx.x;
  double r[kNb];
  const double *src = A + (j0 + i) * k + j0;
#pragma unroll
  for (int c = 0; c < kNb; ++c) r[c] = src[c];
#pragma unroll
  for (int c = 0; c < kNb; ++c) {
    const double d = sqrt(lane_bcast(r[c], c));
    const double l = i > c ? r[c] / d : (i == c ? d : 0.0);
    r[c] = l;
#pragma unroll
    for (int jj = c + 1; jj < kNb; ++jj) r[jj] = fma(-l, lane_bcast(l, jj), r[jj]);
  }
  double *dst = A + (j0 + i) * k + j0;
#pragma unroll
  for (int c = 0; c < kNb; ++c) dst[c] = c <= i ? r[c] : 0.0;
}

// panel below the diagonal block: rows solve x L11^T = a.  A team of kTeamT
// lanes per row, lane t holding columns [kPerT t, kPerT t + kPerT): step c, the
// owner of column c divides by l_cc and the team takes x_c in one cross-lane
// read; every later column subtracts x_c l[c'][c].  Each x_c' sees the same
// operations in the same order as a lane solving its row alone.
constexpr int kTeamT = 16;
constexpr int kPerT = kNb / kTeamT;
__global__ __launch_bounds__(kThr) void trsm_kernel(double *__restrict__ A, int64_t k, int64_t j0) {
  __shared__ double l[kNb][kLdp];
  for (int e = threadIdx.x; e < kNb * kNb; e += kThr)
    l[e / kNb][e % kNb] = A[(j0 + e / kNb) * k + j0 + e % kNb];
  __syncthreads();
  const int t = threadIdx.x % kTeamT;
  const int64_t r = j0 + kNb + (int64_t)blockIdx.x * (kThr / kTeamT) + threadIdx.x / kTeamT;
  const bool live = r < k;
  const int64_t rr = live ? r : k - 1;   // a row below the block (launched only when rows remain)
  double x[kPerT];
#pragma unroll
  for (int c = 0; c < kPerT; ++c) x[c] = A[rr * k + j0 + kPerT * t + c];
#pragma unroll
  for (int c = 0; c < kNb; ++c) {
    const int owner = c / kPerT, lc = c % kPerT;
    const double xc = __shfl(x[lc] / l[c][c], owner, kTeamT);
    if (t == owner) x[lc] = xc;
#pragma unroll
    for (int jj = 0; jj < kPerT; ++jj)
      if (kPerT * t + jj > c) x[jj] = fma(-xc, l[kPerT * t + jj][c], x[jj]);
  }
  if (live) {
#pragma unroll
    for (int c = 0; c < kPerT; ++c) A[rr * k + j0 + kPerT * t + c] = x[c];
  }
}

// C -= P_i P_j^T on the trailing lower tiles, P = A[r0:, j0:j0+64]
__global__ __launch_bounds__(kThr) void syrk_kernel(double *__restrict__ A, int64_t k, int64_t j0) {
  const int ti = blockIdx.y, tj = blockIdx.x;
  if (tj > ti) return;
  constexpr int H = kNb / 2;   // the 64 inner terms in two LDS halves
  __shared__ double pi[kNb][H + 1], pj[kNb][H + 1];
  const int64_t r0 = j0 + kNb;
  const int64_t i0 = r0 + (int64_t)ti * kNb, c0 = r0 + (int64_t)tj * kNb;
  const int ty = threadIdx.x / 16, tx = threadIdx.x % 16;
  double acc[4][4] = {};
  for (int h = 0; h < 2; ++h) {
    __syncthreads();
    for (int e = threadIdx.x; e < kNb * H; e += kThr) {
      pi[e / H][e % H] = A[(i0 + e / H) * k + j0 + h * H + e % H];
      pj[e / H][e % H] = A[(c0 + e / H) * k + j0 + h * H + e % H];
    }
    __syncthreads();
    for (int p = 0; p < H; ++p) {
      double av[4], bv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) av[u] = pi[ty * 4 + u][p];
#pragma unroll
      for (int v = 0; v < 4; ++v) bv[v] = pj[tx * 4 + v][p];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][v] = fma(av[u], bv[v], acc[u][v]);
    }
  }
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) A[(i0 + ty * 4 + u) * k + c0 + tx * 4 + v] -= acc[u][v];
}

// inverse of every 64 x 64 lower diagonal block of L into Dinv[b] (one
// workgroup each; lane c solves L y = e_c by forward substitution)
__global__ __launch_bounds__(kNb) void diag_inv_kernel(const double *__restrict__ L, int64_t k,
                                                       double *__restrict__ Dinv) {
  __shared__ double l[kNb][kNb], y[kNb][kNb];
  const int64_t b0 = (int64_t)blockIdx.x * kNb;
  for (int e = threadIdx.x; e < kNb * kNb; e += kNb)
    l[e / kNb][e % kNb] = L[(b0 + e / kNb) * k + b0 + e % kNb];
  __syncthreads();
  const int c = threadIdx.x;
  for (int r = 0; r < kNb; ++r) {
    if (r < c) {
      y[r][c] = 0.0;
      continue;
    }
    double s = r == c ? 1.0 : 0.0;
    for (int p = c; p < r; ++p) s -= l[r][p] * y[p][c];
    y[r][c] = s / l[r][r];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < kNb * kNb; e += kNb)
    Dinv[(int64_t)blockIdx.x * kNb * kNb + e] = y[e / kNb][e % kNb];
}

// L^-1 by right-looking block substitution of L X = I, in place in X (which
// holds the running right-hand side, zero below the diagonal at the start).
// Step b: X[b][c] = Dinv_b X[b][c] for c < b and X[b][b] = Dinv_b (inv_scale),
// then X[i][c] -= L[i][b] X[b][c] for every i > b, c <= b (inv_update).

// 64 x 64 tile product acc += P Q, P and Q row-major with leading dimensions,
// through LDS in two halves of the inner dimension (4 x 4 outputs per lane).
__device__ __forceinline__ void tile_mac(const double *__restrict__ P, int64_t ldp,
                                         const double *__restrict__ Q, int64_t ldq,
                                         double (&acc)[4][4], double (*ta)[kNb / 2 + 1],
                                         double (*tb)[kNb + 1]) {
  constexpr int H = kNb / 2;
  const int ty = threadIdx.x / 16, tx = threadIdx.x % 16;
  for (int h = 0; h < 2; ++h) {
    __syncthreads();
    for (int e = threadIdx.x; e < kNb * H; e += kThr) {
      ta[e / H][e % H] = P[(int64_t)(e / H) * ldp + h * H + e % H];
      tb[e / kNb][e % kNb] = Q[(int64_t)(h * H + e / kNb) * ldq + e % kNb];
    }
    __syncthreads();
    for (int q = 0; q < H; ++q) {
      double av[4], bv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) av[u] = ta[ty * 4 + u][q];
#pragma unroll
      for (int v = 0; v < 4; ++v) bv[v] = tb[q][tx * 4 + v];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][v] = fma(av[u], bv[v], acc[u][v]);
    }
  }
}

__global__ __launch_bounds__(kThr) void inv_scale_kernel(const double *__restrict__ Dinv,
                                                         double *__restrict__ X, int64_t k,
                                                         int64_t b) {
  __shared__ double ta[kNb][kNb / 2 + 1], tb[kNb / 2][kNb + 1];
  const int64_t c = blockIdx.x;
  const double *D = Dinv + b * kNb * kNb;
  double *out = X + b * kNb * k + c * kNb;
  const int ty = threadIdx.x / 16, tx = threadIdx.x % 16;
  if (c == b) {
    for (int e = threadIdx.x; e < kNb * kNb; e += kThr) out[(e / kNb) * k + e % kNb] = D[e];
    return;
  }
  double acc[4][4] = {};
  tile_mac(D, kNb, out, k, acc, ta, tb);
  __syncthreads();   // every lane has read the block before it is overwritten
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) out[(ty * 4 + u) * k + tx * 4 + v] = acc[u][v];
}

__global__ __launch_bounds__(kThr) void inv_update_kernel(const double *__restrict__ L,
                                                          double *__restrict__ X, int64_t k,
                                                          int64_t b) {
  __shared__ double ta[kNb][kNb / 2 + 1], tb[kNb / 2][kNb + 1];
  const int64_t c = blockIdx.x, i = b + 1 + blockIdx.y;
  const int ty = threadIdx.x / 16, tx = threadIdx.x % 16;
  double acc[4][4] = {};
  tile_mac(L + i * kNb * k + b * kNb, k, X + b * kNb * k + c * kNb, k, acc, ta, tb);
  double *out = X + i * kNb * k + c * kNb;
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) out[(ty * 4 + u) * k + tx * 4 + v] -= acc[u][v];
}

__global__ __launch_bounds__(kThr) void zero_kernel(double *__restrict__ p, int64_t n) {
  const int64_t e = (int64_t)blockIdx.x * kThr + threadIdx.x;
  if (e < n) p[e] = 0.0;
}

// U[i][j] = X[k-1-i][k-1-j] for j >= i (fp32 for the column loop; fp64 copy on request)
__global__ __launch_bounds__(kThr) void u_kernel(const double *__restrict__ X, int64_t k,
                                                 float *__restrict__ Uf, double *__restrict__ Ud) {
  const int64_t e = (int64_t)blockIdx.x * kThr + threadIdx.x;
  if (e >= k * k) return;
  const int64_t i = e / k, j = e % k;
  const double u = j >= i ? X[(k - 1 - i) * k + (k - 1 - j)] : 0.0;
  Uf[e] = (float)u;
  if (Ud) Ud[e] = u;
}

__device__ __forceinline__ float clampq(float v, float maxq) {
  v = v < 0.0f ? 0.0f : v;
  return v > maxq ? maxq : v;
}

// Group g (columns i1 = 128 g ...): a team of kTeam lanes per weight row,
// lane t of a team holding the group's columns [kPer t, kPer t + kPer) in
// registers; the group's block of U sits in LDS.  Step i: the owner of column
// i quantizes it, its error e_i goes to the team in one cross-lane read, and
// every later column j takes w_j = fma(-e_i, U[i][j], w_j), the same operations
// in the same order as one lane doing the whole row.
constexpr int kTeam = 16;
constexpr int kPer = kGroup / kTeam;   // columns per lane
constexpr int kRowsPerBlock = kThr / kTeam;

template <int BITS>
__global__ __launch_bounds__(kThr) void gptq_group_kernel(
    float *__restrict__ Wk, const float *__restrict__ Uf, int64_t n, int64_t k, int64_t g,
    uint32_t *__restrict__ codes, float *__restrict__ scales, uint8_t *__restrict__ zeros,
    float *__restrict__ err) {
  __shared__ __attribute__((aligned(16))) float ub[kGroup][kGroup];   // U block of the group
  __shared__ uint8_t qs[kRowsPerBlock][kGroup];                       // codes, for packing
  const int64_t i1 = g * kGroup;
  for (int e = threadIdx.x; e < kGroup * kGroup / 4; e += kThr) {
    const int row = e / (kGroup / 4), c4 = e % (kGroup / 4);
    reinterpret_cast<float4 *>(&ub[row][0])[c4] =
        reinterpret_cast<const float4 *>(Uf + (i1 + row) * k + i1)[c4];
  }
  const int t = threadIdx.x % kTeam, tr = threadIdx.x / kTeam;
  const int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + tr;
  const bool live = r < n;
  const int64_t rr = live ? r : n - 1;   // a team past the last row works on a valid row, stores nothing
  const float maxq = (float)((1 << BITS) - 1);
  float w[kPer];
  {
    const float4 *src = reinterpret_cast<const float4 *>(Wk + rr * k + i1 + kPer * t);
#pragma unroll
    for (int i = 0; i < kPer / 4; ++i) {
      const float4 v = src[i];
      w[4 * i] = v.x;
      w[4 * i + 1] = v.y;
      w[4 * i + 2] = v.z;
      w[4 * i + 3] = v.w;
    }
  }
  // the plain quantizer's steps on the group's current weights (min and max
  // over the team: exact in any order)
  float lo = 0.0f, hi = 0.0f;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    lo = w[i] < lo ? w[i] : lo;
    hi = w[i] > hi ? w[i] : hi;
  }
#pragma unroll
  for (int o = kTeam / 2; o > 0; o /= 2) {
    const float l2 = __shfl_xor(lo, o, kTeam), h2 = __shfl_xor(hi, o, kTeam);
    lo = l2 < lo ? l2 : lo;
    hi = h2 > hi ? h2 : hi;
  }
  float s = (hi - lo) / maxq, zf;
  if (s == 0.0f) {
    s = 1.0f;
    zf = 0.0f;
  } else {
    zf = clampq(rintf((-lo) / s), maxq);
  }
  __syncthreads();   // U block staged
  float ev[kPer], qv[kPer];
#pragma unroll
  for (int i = 0; i < kGroup; ++i) {
    const int owner = i / kPer, li = i % kPer;
    // every lane evaluates its own column li; the owner's value is the one used
    const float wi = w[li];
    const float q = clampq(rintf(wi / s) + zf, maxq);
    const float what = (float)((int)q - (int)zf) * s;
    const float ei = (wi - what) / ub[i][i];
    const float e = __shfl(ei, owner, kTeam);
    if (t == owner) {
      ev[li] = ei;
      qv[li] = q;
    }
    if (i + 1 < kGroup) {
      const float4 u0 = *reinterpret_cast<const float4 *>(&ub[i][kPer * t]);
      const float4 u1 = *reinterpret_cast<const float4 *>(&ub[i][kPer * t + 4]);
      const float u[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
      for (int jj = 0; jj < kPer; ++jj)
        if (kPer * t + jj > i) w[jj] = fmaf(-e, u[jj], w[jj]);
    }
  }
  static_assert(kPer == 8, "the U row slice is read as two float4");
  // errors and codes of this lane's columns
  if (live) {
    float4 *er = reinterpret_cast<float4 *>(err + rr * kGroup + kPer * t);
    er[0] = make_float4(ev[0], ev[1], ev[2], ev[3]);
    er[1] = make_float4(ev[4], ev[5], ev[6], ev[7]);
  }
#pragma unroll
  for (int jj = 0; jj < kPer; ++jj) qs[tr][kPer * t + jj] = (uint8_t)(int)qv[jj];
  __syncthreads();
  // pack: lane t writes words t and t + kTeam of the row's 4 * BITS words
  // (32-code chunks of BITS words, code j of a chunk at bit j * BITS)
  if (live) {
    uint32_t *dst = codes + rr * (k * BITS / 32) + g * 4 * BITS;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int W = t + kTeam * h;
      if (W >= 4 * BITS) continue;
      const int c = W / BITS, wd = W % BITS;
      uint32_t out = 0u;
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const int lo_bit = j * BITS - 32 * wd;
        if (lo_bit <= -BITS || lo_bit >= 32) continue;
        const uint32_t q = qs[tr][32 * c + j];
        out |= lo_bit >= 0 ? q << lo_bit : q >> (-lo_bit);
      }
      dst[W] = out;
    }
    if (t == 0) {
      const int64_t G = k / kGroup;
      scales[rr * G + g] = s;
      zeros[rr * G + g] = (uint8_t)(int)zf;
    }
  }
}

// Wk[:, c] -= sum_p err[:, p] U[i1 + p][c] for the columns after group g:
// 128 x 128 output tiles, 8 x 8 per thread, the 128 inner terms in two LDS
// halves (errors transposed to [p][row]); each output accumulates its terms in
// p order.
constexpr int kUpT = 128, kUpP = 64;
__global__ __launch_bounds__(kThr) void gptq_update_kernel(float *__restrict__ Wk,
                                                           const float *__restrict__ Uf,
                                                           const float *__restrict__ err,
                                                           int64_t n, int64_t k, int64_t g) {
  __shared__ __attribute__((aligned(16))) float ta[kUpP][kUpT];   // err^T half: [p][row]
  __shared__ __attribute__((aligned(16))) float tb[kUpP][kUpT];   // U half: [p][column]
  const int64_t i1 = g * kGroup, c0 = i1 + kGroup + (int64_t)blockIdx.y * kUpT;
  const int64_t r0 = (int64_t)blockIdx.x * kUpT;
  const int ty = threadIdx.x / 16, tx = threadIdx.x % 16;
  float acc[8][8];
#pragma unroll
  for (int u = 0; u < 8; ++u)
#pragma unroll
    for (int v = 0; v < 8; ++v) acc[u][v] = 0.0f;
  for (int h = 0; h < kGroup / kUpP; ++h) {
    if (h) __syncthreads();   // the previous half is consumed
    // errors: thread e takes row e % 128 and terms 4 (e / 128) .. + 3
    for (int e = threadIdx.x; e < kUpT * kUpP / 4; e += kThr) {
      const int rr = e % kUpT, p4 = e / kUpT;
      const int64_t row = r0 + rr;
      const float4 v = row < n ? *reinterpret_cast<const float4 *>(err + row * kGroup + h * kUpP + 4 * p4)
                               : make_float4(0.f, 0.f, 0.f, 0.f);
      ta[4 * p4 + 0][rr] = v.x;
      ta[4 * p4 + 1][rr] = v.y;
      ta[4 * p4 + 2][rr] = v.z;
      ta[4 * p4 + 3][rr] = v.w;
    }
    // U rows i1 + 64 h + p, columns c0 .. c0 + 127 (the later columns come in whole tiles)
    for (int e = threadIdx.x; e < kUpP * kUpT / 4; e += kThr) {
      const int pp = e / (kUpT / 4), c4 = e % (kUpT / 4);
      *reinterpret_cast<float4 *>(&tb[pp][4 * c4]) =
          *reinterpret_cast<const float4 *>(Uf + (i1 + h * kUpP + pp) * k + c0 + 4 * c4);
    }
    __syncthreads();
#pragma unroll 4
    for (int pp = 0; pp < kUpP; ++pp) {
      const float4 a0 = *reinterpret_cast<const float4 *>(&ta[pp][8 * ty]);
      const float4 a1 = *reinterpret_cast<const float4 *>(&ta[pp][8 * ty + 4]);
      const float4 b0 = *reinterpret_cast<const float4 *>(&tb[pp][8 * tx]);
      const float4 b1 = *reinterpret_cast<const float4 *>(&tb[pp][8 * tx + 4]);
      const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
      const float bv[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int v = 0; v < 8; ++v) acc[u][v] = fmaf(av[u], bv[v], acc[u][v]);
    }
  }
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int64_t row = r0 + 8 * ty + u;
    if (row >= n) continue;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      float4 *dst = reinterpret_cast<float4 *>(Wk + row * k + c0 + 8 * tx + 4 * q);
      float4 w = *dst;
      w.x -= acc[u][4 * q];
      w.y -= acc[u][4 * q + 1];
      w.z -= acc[u][4 * q + 2];
      w.w -= acc[u][4 * q + 3];
      *dst = w;
    }
  }
}

template <int BITS>
hipError_t group_launch(float *Wk, const float *Uf, int64_t n, int64_t k, int64_t g,
                        uint32_t *codes, float *scales, uint8_t *zeros, float *err,
                        hipStream_t s) {
  hipLaunchKernelGGL((gptq_group_kernel<BITS>), dim3((unsigned)((n + kRowsPerBlock - 1) / kRowsPerBlock)),
                     dim3(kThr), 0, s, Wk, Uf, n, k, g, codes, scales, zeros, err);
  return hipGetLastError();
}

}  // namespace

// Factor workspace: A, X fp64 [k][k] | stat (256 B) | Dinv fp64 [k/64][64][64].
size_t gptq_factor_workspace(int64_t k) {
  const size_t b = (size_t)k * k * 8 * 2 + 256 + (size_t)k * kNb * 8;
  return (b + 255) / 256 * 256;
}

// Column-pass workspace: Wk fp32 [n][k] | err fp32 [n][128].
size_t gptq_columns_workspace(int64_t n, int64_t k) {
  const size_t b = (size_t)n * k * 4 + (size_t)n * kGroup * 4;
  return (b + 255) / 256 * 256;
}

// Whole pipeline: Uf fp32 [k][k] | dead [k] (256-byte padded) | factor | column pass.
size_t gptq_workspace(int64_t n, int64_t k) {
  const size_t uf = (size_t)k * k * 4, dead = ((size_t)k + 255) / 256 * 256;
  return uf + dead + gptq_factor_workspace(k) + gptq_columns_workspace(n, k);
}

hipError_t launch_gptq_factor(const float *H, int64_t k, double damp, float *Uf, uint8_t *dead,
                              double *u_out, void *ws, hipStream_t s) {
  double *A = static_cast<double *>(ws);
  double *X = A + k * k;
  double *stat = X + k * k;                // 256 bytes
  double *Dinv = stat + 32;                // [k / 64][64][64]
  hipError_t e;
  const unsigned kk = (unsigned)((k * k + kThr - 1) / kThr);
  hipLaunchKernelGGL(diag_mean_kernel, dim3(1), dim3(kThr), 0, s, H, k, stat, dead);
  hipLaunchKernelGGL(prep_kernel, dim3(kk), dim3(kThr), 0, s, H, k, damp, stat, A);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t nbk = k / kNb;
  for (int64_t b = 0; b < nbk; ++b) {
    const int64_t j0 = b * kNb;
    hipLaunchKernelGGL(potf2_kernel, dim3(1), dim3(kNb), 0, s, A, k, j0);
    const int64_t rest = k - j0 - kNb;
    if (rest > 0) {
      hipLaunchKernelGGL(trsm_kernel, dim3((unsigned)((rest + kThr / kTeamT - 1) / (kThr / kTeamT))),
                         dim3(kThr), 0, s, A, k, j0);
      const unsigned t = (unsigned)(rest / kNb);
      hipLaunchKernelGGL(syrk_kernel, dim3(t, t), dim3(kThr), 0, s, A, k, j0);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(diag_inv_kernel, dim3((unsigned)nbk), dim3(kNb), 0, s, A, k, Dinv);
  hipLaunchKernelGGL(zero_kernel, dim3(kk), dim3(kThr), 0, s, X, k * k);
  for (int64_t b = 0; b < nbk; ++b) {
    hipLaunchKernelGGL(inv_scale_kernel, dim3((unsigned)(b + 1)), dim3(kThr), 0, s, Dinv, X, k, b);
    if (b + 1 < nbk)
      hipLaunchKernelGGL(inv_update_kernel, dim3((unsigned)(b + 1), (unsigned)(nbk - b - 1)),
                         dim3(kThr), 0, s, A, X, k, b);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(u_kernel, dim3(kk), dim3(kThr), 0, s, X, k, Uf, u_out);
  return hipGetLastError();
}

hipError_t launch_gptq_columns(const float *W, const float *Uf, const uint8_t *dead, int64_t n,
                               int64_t k, int bits, uint32_t *codes, float *scales,
                               uint8_t *zeros, void *ws, hipStream_t s) {
  float *Wk = static_cast<float *>(ws);
  float *err = Wk + n * k;
  hipError_t e;
  hipLaunchKernelGGL(wcopy_kernel, dim3((unsigned)((n * k + kThr - 1) / kThr)), dim3(kThr), 0, s,
                     W, dead, n, k, Wk);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t G = k / kGroup;
  for (int64_t g = 0; g < G; ++g) {
    switch (bits) {
      case 2: e = group_launch<2>(Wk, Uf, n, k, g, codes, scales, zeros, err, s); break;
      case 3: e = group_launch<3>(Wk, Uf, n, k, g, codes, scales, zeros, err, s); break;
      case 4: e = group_launch<4>(Wk, Uf, n, k, g, codes, scales, zeros, err, s); break;
      case 5: e = group_launch<5>(Wk, Uf, n, k, g, codes, scales, zeros, err, s); break;
      case 6: e = group_launch<6>(Wk, Uf, n, k, g, codes, scales, zeros, err, s); break;
      case 7: e = group_launch<7>(Wk, Uf, n, k, g, codes, scales, zeros, err, s); break;
      case 8: e = group_launch<8>(Wk, Uf, n, k, g, codes, scales, zeros, err, s); break;
      default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    const int64_t later = k - (g + 1) * kGroup;
    if (later > 0) {
      hipLaunchKernelGGL(gptq_update_kernel,
                         dim3((unsigned)((n + kUpT - 1) / kUpT), (unsigned)(later / kUpT)), dim3(kThr),
                         0, s, Wk, Uf, err, n, k, g);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

hipError_t launch_gptq(const float *W, const float *H, int64_t n, int64_t k, int bits, double damp,
                       uint32_t *codes, float *scales, uint8_t *zeros, double *u_out, void *ws,
                       hipStream_t s) {
  char *p = static_cast<char *>(ws);
  float *Uf = reinterpret_cast<float *>(p);
  uint8_t *dead = reinterpret_cast<uint8_t *>(p + (size_t)k * k * 4);
  char *fws = reinterpret_cast<char *>(dead) + ((size_t)k + 255) / 256 * 256;
  char *cws = fws + gptq_factor_workspace(k);
  hipError_t e = launch_gptq_factor(H, k, damp, Uf, dead, u_out, fws, s);
  if (e != hipSuccess) return e;
  return launch_gptq_columns(W, Uf, dead, n, k, bits, codes, scales, zeros, cws, s);
}

}  // namespace slq
