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

// IEEE binary16 bits -> fp32 (exact).
__device__ __forceinline__ float f16_bits_to_f32(uint32_t bits) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

// The smallest binary16 value >= s (s > 0, finite), as bits: a scale rounded up
// keeps the half-step error bound of the grid it spans.  Values above the
// binary16 range saturate at 65504.
__device__ __forceinline__ uint32_t f16_bits_round_up(float s) {
  uint32_t b = __builtin_bit_cast(uint16_t, (_Float16)s);   // nearest, ties to even
  if (f16_bits_to_f32(b) < s) b += 1u;                       // next value up
  return b >= 0x7C00u ? 0x7BFFu : b;
}

// Group metadata, in one of two layouts (flat group index i = row * G + g):
//  CM = false: fp32 scales[i], zero points as bytes zeros[i];
//  CM = true (20 bits per group for b <= 4): binary16 scales[i] rounded up from
//    the fp32 scale; zero points as 4-bit nibbles (b <= 4: nibble i of the byte
//    stream, low nibble first) or bytes (b >= 5).
template <int BITS, bool CM>
struct MetaRd {
  const void *s;
  const uint8_t *z;
  __device__ __forceinline__ float scale(int64_t i) const {
    if constexpr (CM) return f16_bits_to_f32(static_cast<const uint16_t *>(s)[i]);
    else return static_cast<const float *>(s)[i];
  }
  __device__ __forceinline__ uint32_t zero(int64_t i) const {
    if constexpr (CM && BITS <= 4) return (uint32_t)(z[i >> 1] >> ((i & 1) * 4)) & 15u;
    else return z[i];
  }
  // groups i..i+3 (i % 4 == 0): scales, and zero points as the bytes of one word
  __device__ __forceinline__ void load4(int64_t i, float4 &sv, uint32_t &zv) const {
    if constexpr (CM) {
      const u32x2_t h = *reinterpret_cast<const u32x2_t *>(static_cast<const uint16_t *>(s) + i);
      sv = make_float4(f16_bits_to_f32(h[0] & 0xFFFFu), f16_bits_to_f32(h[0] >> 16),
                       f16_bits_to_f32(h[1] & 0xFFFFu), f16_bits_to_f32(h[1] >> 16));
      if constexpr (BITS <= 4) {
        const uint32_t v = *reinterpret_cast<const uint16_t *>(z + (i >> 1));
        zv = (v & 0xFu) | ((v & 0xF0u) << 4) | ((v & 0xF00u) << 8) | ((v & 0xF000u) << 12);
      } else {
        zv = *reinterpret_cast<const uint32_t *>(z + i);
      }
    } else {
      sv = *reinterpret_cast<const float4 *>(static_cast<const float *>(s) + i);
      zv = *reinterpret_cast<const uint32_t *>(z + i);
    }
  }
};

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

}  // namespace slq
