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

// ---------------------------------------------------------------------------
// 4-bit code tables.  A table gives the value of each of the 16 codes (fp32
// bits, in code order) and the quantizer's rule: the distinct values in
// ascending order, the decision threshold between consecutive ones, and the
// code written for "x lies above exactly `count` thresholds".
//
// Decision threshold between distinct values v_i < v_{i+1}: their exact
// midpoint (exact in double) rounded toward -inf to fp32.  For an fp32 x,
// x > T_i  <=>  x is strictly nearer to v_{i+1}, so count = #{i : x > T_i}
// picks the nearest value with ties to the lower one.
// ---------------------------------------------------------------------------
constexpr uint32_t midpoint_down_bits(float lo, float hi) {
  double mid = ((double)lo + (double)hi) * 0.5;
  float f = (float)mid;  // round to nearest
  uint32_t b = __builtin_bit_cast(uint32_t, f);
  if ((double)f > mid) {  // step one ulp toward -inf
    if (f > 0.0f) b -= 1u;
    else if (f < 0.0f) b += 1u;
    else b = 0x80000001u;
  }
  return b;
}

struct CodeTable {
  uint32_t level[16];    // value of each code (fp32 bits)
  int ndist;             // distinct values (equal values, e.g. +0 and -0, count once)
  uint32_t dist[16];     // distinct values, ascending (fp32 bits)
  uint8_t dist_code[16]; // code written for distinct value i (the lowest such code)
  uint32_t thr[15];      // ndist - 1 thresholds (fp32 bits)
  uint8_t zero_code;     // code of an all-zero block
};

// Over the first n codes (the others keep value +0 and take no part).
constexpr CodeTable make_code_table(const uint32_t (&lv)[16], int n = 16) {
  CodeTable t{};
  for (int c = 0; c < n; ++c) t.level[c] = lv[c];
  // distinct values in ascending order (selection by value, lowest code wins)
  t.ndist = 0;
  float last = 0.0f;
  for (int k = 0; k < n; ++k) {
    int best = -1;
    for (int c = 0; c < n; ++c) {
      const float v = __builtin_bit_cast(float, lv[c]);
      if (t.ndist > 0 && !(v > last)) continue;
      if (best < 0 || v < __builtin_bit_cast(float, lv[best])) best = c;
    }
    if (best < 0) break;
    last = __builtin_bit_cast(float, lv[best]);
    t.dist[t.ndist] = lv[best];
    t.dist_code[t.ndist] = (uint8_t)best;
    if (last == 0.0f) t.zero_code = (uint8_t)best;
    ++t.ndist;
  }
  for (int i = 0; i + 1 < t.ndist; ++i)
    t.thr[i] = midpoint_down_bits(__builtin_bit_cast(float, t.dist[i]),
                                  __builtin_bit_cast(float, t.dist[i + 1]));
  return t;
}

constexpr bool code_table_sound(const CodeTable& t) {
  for (int i = 0; i + 1 < t.ndist; ++i) {
    const float lo = __builtin_bit_cast(float, t.dist[i]);
    const float hi = __builtin_bit_cast(float, t.dist[i + 1]);
    if (!(lo < hi)) return false;
    const double mid = ((double)lo + (double)hi) * 0.5;
    const float th = __builtin_bit_cast(float, t.thr[i]);
    if (t.thr[i] == 0x80000000u) return false;         // never -0 (+0 for a midpoint of 0)
    if ((double)th > mid) return false;                 // at or below the midpoint
    const uint32_t nb = t.thr[i] + ((th >= 0.0f) ? 1u : (uint32_t)-1);
    if ((double)__builtin_bit_cast(float, nb) <= mid) return false;  // next float above it
    if (!(lo <= th && th < hi)) return false;
  }
  return true;
}

// FP4: the E2M1 format (bit 3 sign, bits 2..1 exponent with bias 1, bit 0
// mantissa; exponent 0 is subnormal), magnitudes 0, 1/2, 1, 3/2, 2, 3, 4, 6,
// divided by 6 so that the largest magnitude is 1 like the NF4 levels, and
// rounded once to fp32.  Code 8 is -0.
constexpr uint32_t fp4_level_bits(int c) {
  const int e = (c >> 1) & 3, m = c & 1;
  const double mag = (e == 0) ? 0.5 * m : (double)(1 << (e - 1)) * (1.0 + 0.5 * m);
  const float v = (float)(mag / 6.0);
  return __builtin_bit_cast(uint32_t, (c & 8) ? -v : v);
}
struct Fp4Bits {
  uint32_t b[16];
  constexpr Fp4Bits() : b{} {
    for (int c = 0; c < 16; ++c) b[c] = fp4_level_bits(c);
  }
};
constexpr Fp4Bits kFp4Bits{};

// k-bit NormalFloat for k = 3 and 2 (the ModuLoRA abstract finetunes through
// 2-, 3- and 4-bit weights): 2^k levels built the NF4 way, with an exact
// zero, 2^(k-1) positive and 2^(k-1) - 1 negative levels at evenly spaced
// normal probabilities up to delta_k = 1 - (1/(2(2^k-1)) + 1/2^(k+1)) / 2,
// divided by Phi^{-1}(delta_k) and rounded once to fp32 (bits from scipy's
// ndtri; every value sits more than 5e-9 relative from an fp32 rounding
// boundary).  The 16-entry tables are padded with +0 past 2^k codes.
constexpr uint32_t kNf3Bits[16] = {0xbf800000u, 0xbf08f740u, 0xbe7cdb98u, 0x00000000u,
                                   0x3e3bbcd2u, 0x3ec394b6u, 0x3f1f7bfeu, 0x3f800000u};
constexpr uint32_t kNf2Bits[16] = {0xbf800000u, 0x00000000u, 0x3edf238fu, 0x3f800000u};

// Each code type also gives the code for a threshold count in closed form
// (checked against the table below) and its width in bits.
struct CodeNF4 {
  static constexpr bool kUser = false;
  static constexpr int kId = 0;
  static constexpr int kBits = 4;
  static constexpr CodeTable table = make_code_table(kLevelBits);
  __host__ __device__ static constexpr uint32_t code_of_count(uint32_t n) { return n; }
};
struct CodeNF3 {
  static constexpr bool kUser = false;
  static constexpr int kId = 2;
  static constexpr int kBits = 3;
  static constexpr CodeTable table = make_code_table(kNf3Bits);
  __host__ __device__ static constexpr uint32_t code_of_count(uint32_t n) { return n; }
};
struct CodeNF2 {
  static constexpr bool kUser = false;
  static constexpr int kId = 3;
  static constexpr int kBits = 2;
  static constexpr CodeTable table = make_code_table(kNf2Bits);
  __host__ __device__ static constexpr uint32_t code_of_count(uint32_t n) { return n; }
};
struct CodeFP4 {
  static constexpr bool kUser = false;
  static constexpr int kId = 1;
  static constexpr int kBits = 4;
  static constexpr CodeTable table = make_code_table(kFp4Bits.b);
  // counts 0..6 are -1 .. -1/12 (codes 15..9), 7 is zero (code 0), 8..14 are
  // 1/12 .. 1 (codes 1..7)
  __host__ __device__ static constexpr uint32_t code_of_count(uint32_t n) {
    return n >= 7 ? n - 7 : 15 - n;
  }
};
template <class CT>
constexpr bool count_map_sound() {
  for (int n = 0; n < CT::table.ndist; ++n)
    if (CT::code_of_count((uint32_t)n) != CT::table.dist_code[n]) return false;
  return true;
}
static_assert(count_map_sound<CodeNF4>() && count_map_sound<CodeFP4>() &&
                  count_map_sound<CodeNF3>() && count_map_sound<CodeNF2>(),
              "count -> code maps");
static_assert(CodeNF3::table.ndist == 8 && CodeNF3::table.zero_code == 3 &&
                  code_table_sound(CodeNF3::table),
              "NF3: 8 distinct levels, zero is code 3");
static_assert(CodeNF2::table.ndist == 4 && CodeNF2::table.zero_code == 1 &&
                  code_table_sound(CodeNF2::table),
              "NF2: 4 distinct levels, zero is code 1");
static_assert(CodeNF4::table.ndist == 16 && CodeNF4::table.zero_code == 7 &&
                  code_table_sound(CodeNF4::table),
              "NF4: 16 distinct levels, zero is code 7, thresholds are the midpoints rounded down");
static_assert(CodeFP4::table.ndist == 15 && CodeFP4::table.zero_code == 0 &&
                  code_table_sound(CodeFP4::table),
              "FP4: 15 distinct values (+0 and -0), zero is code 0");

template <class CT>
__host__ __device__ constexpr float code_value(int c) {
  return __builtin_bit_cast(float, CT::table.level[c]);
}

// ---------------------------------------------------------------------------
// A caller's codebook (the ModuLoRA abstract finetunes through weights
// materialized from a black-box quantizer: any 2^k values behind the codes).
// The values and the quantizer's rule are derived on the host with the same
// construction as the built-in tables (make_code_table over the first 2^k
// codes) and travel by value in the kernel arguments, so the code words stay
// uniform (scalar registers).
// ---------------------------------------------------------------------------
struct UserTable {
  float level[16];    // value of each code (0 past 2^k)
  float thr[15];      // decision thresholds ascending; +inf past the last
  uint32_t code_lo;   // code for threshold count n: nibble n of code_hi:code_lo
  uint32_t code_hi;
};

template <int K, int Id>
struct CodeUser {
  static constexpr bool kUser = true;
  static constexpr int kId = Id;
  static constexpr int kBits = K;
};
using CodeUser4 = CodeUser<4, 4>;
using CodeUser3 = CodeUser<3, 5>;
using CodeUser2 = CodeUser<2, 6>;

// Value of code c: the built-in table, or the caller's.
template <class CT>
__host__ __device__ __forceinline__ float level_of(const UserTable& u, int c) {
  if constexpr (CT::kUser) return u.level[c];
  else return code_value<CT>(c);
}

// Call f(CT{}) for the code type with this id (NF4 for an unknown id; the C
// ABI rejects unknown ids before any launch).
template <class F>
__host__ auto with_code(int id, F&& f) {
  switch (id) {
    case CodeFP4::kId: return f(CodeFP4{});
    case CodeNF3::kId: return f(CodeNF3{});
    case CodeNF2::kId: return f(CodeNF2{});
    default: return f(CodeNF4{});
  }
}

// with_code, also for the caller-codebook types.
template <class F>
__host__ auto with_any_code(int id, F&& f) {
  switch (id) {
    case CodeUser4::kId: return f(CodeUser4{});
    case CodeUser3::kId: return f(CodeUser3{});
    case CodeUser2::kId: return f(CodeUser2{});
    default: return with_code(id, f);
  }
}

// ---------------------------------------------------------------------------
// Packed codes.  A 64-element block takes 8 k bytes (k = bits per code), as
// two halves of 4 k bytes (k little-endian words) for elements 0..31 and
// 32..63.  4 bits: element 2j of the block in the low nibble of byte j.
// 3 and 2 bits: within a half, element 8 g + 2 i + p (g, i in 0..3, p in
// 0..1) has code bits 0-1 at bit 8 i + 2 g of word p and, for 3 bits, code
// bit 2 at bit (8 i + 2 + 2 g + p) mod 32 of word 2.  Every kernel loads a
// half's words and expands each group of eight codes into one word of eight
// nibbles (element order), which is the 4-bit layout, just before its
// table lookup.
// ---------------------------------------------------------------------------
template <int kBits>
struct HalfRaw {
  uint32_t w[kBits];
};

template <class CT>
__host__ __device__ constexpr int64_t block_bytes() {
  return 8 * CT::kBits;
}
template <class CT>
__host__ __device__ constexpr int64_t half_bytes() {
  return 4 * CT::kBits;
}

// The words of one half block at p (4-byte aligned; 16-byte aligned for
// 4 bits, 8-byte aligned for 2 bits).
template <class CT>
__device__ __forceinline__ HalfRaw<CT::kBits> load_half(const uint8_t* p) {
  HalfRaw<CT::kBits> r;
  if constexpr (CT::kBits == 4) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(p);
    r.w[0] = v[0]; r.w[1] = v[1]; r.w[2] = v[2]; r.w[3] = v[3];
  } else if constexpr (CT::kBits == 2) {
    const u32x2 v = *reinterpret_cast<const u32x2*>(p);
    r.w[0] = v[0]; r.w[1] = v[1];
  } else {
    const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
    r.w[0] = q[0]; r.w[1] = q[1]; r.w[2] = q[2];
  }
  return r;
}

// The same words through a buffer resource: byte offset voff (per lane)
// plus soff (uniform).  Out-of-range words read as 0.
template <class CT>
__device__ __forceinline__ HalfRaw<CT::kBits> load_half(__amdgpu_buffer_rsrc_t rsrc, int voff,
                                                        int soff) {
  HalfRaw<CT::kBits> r;
  if constexpr (CT::kBits == 4) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff, soff, 0);
    r.w[0] = v[0]; r.w[1] = v[1]; r.w[2] = v[2]; r.w[3] = v[3];
  } else if constexpr (CT::kBits == 2) {
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rsrc, voff, soff, 0);
    r.w[0] = v[0]; r.w[1] = v[1];
  } else {
    typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
    const u32x3 v = __builtin_amdgcn_raw_buffer_load_b96(rsrc, voff, soff, 0);
    r.w[0] = v[0]; r.w[1] = v[1]; r.w[2] = v[2];
  }
  return r;
}

// A buffer resource over `bytes` bytes at p (the caller keeps bytes below
// 2^31, so every offset fits the 32-bit offset fields).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t bytes_rsrc(const void* p, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                           0x00020000);
}

// Codes 8 g .. 8 g + 7 of a half as eight nibbles (element 8 g + j in
// nibble j).
template <class CT>
__device__ __forceinline__ uint32_t nibbles(const HalfRaw<CT::kBits>& r, int g) {
  if constexpr (CT::kBits == 4) {
    return r.w[g];
  } else {
    uint32_t e = (r.w[0] >> (2 * g)) & 0x03030303u;  // codes of elements 8 g + 2 i
    uint32_t o = (r.w[1] >> (2 * g)) & 0x03030303u;  // codes of elements 8 g + 2 i + 1
    if constexpr (CT::kBits == 3) {
      e |= __builtin_amdgcn_alignbit(r.w[2], r.w[2], 2 * g) & 0x04040404u;
      o |= __builtin_amdgcn_alignbit(r.w[2], r.w[2], 2 * g + 1) & 0x04040404u;
    }
    return e | (o << 4);
  }
}

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
