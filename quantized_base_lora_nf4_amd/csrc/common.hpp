// Shared device helpers for the NF4 + LoRA kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// NF4 levels.  16 values at normal quantiles with an exact zero, normalized to
// [-1, 1] ("QLoRA: fine-tuning a 65B model on one GPU", section "NormalFloat,
// double quantization, paged optimizers").  The probabilities behind them
// are delta - (delta - 1/2) i / 8 (i = 0..7) on the positive side and
// delta - (delta - 1/2) j / 7 (j = 0..6) mirrored on the negative side, with
// delta = 1 - (1/30 + 1/32) / 2; each quantile is divided by Phi^{-1}(delta)
// and rounded once to fp32.  Stored here as fp32 bit patterns, ascending.
// ---------------------------------------------------------------------------
constexpr uint32_t kLevelBits[16] = {
    0xbf800000u, 0xbf3239b1u, 0xbf066b2eu, 0xbeca329eu, 0xbe91a24bu, 0xbe3d353du,
    0xbdba7869u, 0x00000000u, 0x3da2fb01u, 0x3e24cadfu, 0x3e7c04dau, 0x3ead0336u,
    0x3ee1a4b5u, 0x3f1007a9u, 0x3f3913b0u, 0x3f800000u};

constexpr float level_f32(int i) { return __builtin_bit_cast(float, kLevelBits[i]); }

// Decision threshold between level i and level i + 1: their exact midpoint
// (exact in double) rounded toward -inf to fp32.  For an fp32 x,
// x > T_i  <=>  x is strictly nearer to level i + 1, so
// code = #{i : x > T_i} is the nearest level with ties to the lower one.
constexpr uint32_t threshold_bits(int i) {
  double mid = ((double)level_f32(i) + (double)level_f32(i + 1)) * 0.5;
  float f = (float)mid;  // round to nearest
  uint32_t b = __builtin_bit_cast(uint32_t, f);
  if ((double)f > mid) {  // step one ulp toward -inf
    if (f > 0.0f) b -= 1u;
    else if (f < 0.0f) b += 1u;
    else b = 0x80000001u;
  }
  return b;
}

struct ThresholdTable {
  uint32_t bits[15];
  constexpr ThresholdTable() : bits{} {
    for (int i = 0; i < 15; ++i) bits[i] = threshold_bits(i);
  }
};
constexpr ThresholdTable kThr{};

constexpr bool thresholds_sound() {
  for (int i = 0; i < 15; ++i) {
    double mid = ((double)level_f32(i) + (double)level_f32(i + 1)) * 0.5;
    float t = __builtin_bit_cast(float, kThr.bits[i]);
    if ((double)t > mid) return false;                       // at or below mid
    uint32_t nb = kThr.bits[i] + ((t >= 0.0f) ? 1u : (uint32_t)-1);
    if (t == 0.0f) return false;
    float nx = __builtin_bit_cast(float, nb);
    if ((double)nx <= mid) return false;                     // next float above mid
    if (!(level_f32(i) <= t && t < level_f32(i + 1))) return false;
  }
  return true;
}
static_assert(thresholds_sound(), "NF4 thresholds must be the midpoints rounded down");

// ---------------------------------------------------------------------------
// bf16 helpers
// ---------------------------------------------------------------------------

// Round two fp32 values to bf16 (nearest, ties to even) and pack them, `lo`
// in bits 0..15.  Lowers to one v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 r = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float bf16_lo_to_f32(uint32_t v) {
  return __builtin_bit_cast(float, v << 16);
}
__device__ __forceinline__ float bf16_hi_to_f32(uint32_t v) {
  return __builtin_bit_cast(float, v & 0xffff0000u);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t v) {
  return __builtin_bit_cast(float, ((uint32_t)v) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  return (uint16_t)(pack_bf16x2(x, 0.0f) & 0xffffu);
}

// ---------------------------------------------------------------------------
// MFMA wrappers (bf16 in, fp32 accumulate)
// ---------------------------------------------------------------------------

// D[32x32] += A[32x16] * B[16x32].  Lane l supplies A[l % 32][8 (l / 32) + e]
// and B[8 (l / 32) + e][l % 32] for e = 0..7, and holds
// D[8 (v / 4) + 4 (l / 32) + v % 4][l % 32] in element v of the result.
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// D[16x16] += A[16x32] * B[32x16].  Lane l supplies A[l % 16][8 (l / 16) + e]
// and B[8 (l / 16) + e][l % 16], and holds D[4 (l / 16) + v][l % 16].
__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) {
  return __builtin_bit_cast(bf16x8, v);
}

}  // namespace qn
