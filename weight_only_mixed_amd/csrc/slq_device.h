// Device-side helpers shared by the gfx950 kernels of libslq.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

namespace slq {

constexpr int kGroup = 128;        // quantization group along k
constexpr int kWave = 64;          // CDNA wavefront

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

// 16x16x32 bf16 MFMA: D[16x16] += A[16x32] * B[32x16], fp32 accumulate.
// Lane l supplies A row (l % 16) and B column (l % 16), k slots 8*(l/16)+t;
// it receives D rows 4*(l/16)+v, column l % 16, v = 0..3.
__device__ __forceinline__ f32x4_t mfma16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// Byte permute: bytes 0..3 come from `lo`, 4..7 from `hi`.
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// ({hi,lo} >> s)[31:0]
__device__ __forceinline__ uint32_t alignbit(uint32_t hi, uint32_t lo, uint32_t s) {
  return __builtin_amdgcn_alignbit(hi, lo, s);
}

// Selector for perm() that builds {h16 of `hi` word half hh, l16 of `lo` word half lh}.
__host__ __device__ constexpr uint32_t halves_sel(int lh, int hh) {
  return (uint32_t)(2 * lh) | (uint32_t)(2 * lh + 1) << 8 | (uint32_t)(4 + 2 * hh) << 16 |
         (uint32_t)(4 + 2 * hh + 1) << 24;
}

// The value of `v`, held in a VGPR the compiler cannot constant-fold.  gfx9
// VOP3 encodings take no literal operand, so a mask/offset pair of literals
// would split v_and_or_b32 into v_and + v_or; one operand in a register keeps
// the three-input form.
__device__ __forceinline__ uint32_t in_vgpr(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

}  // namespace slq
