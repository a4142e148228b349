// Block quantizer (NF4, FP4, NF3 or NF2 code table) with double-quantized
// absmax constants, and the standalone dequantizer.
//
// Quantization follows "QLoRA: fine-tuning a 65B model on one GPU", section
// "NormalFloat, double quantization, paged optimizers" (16 levels at normal
// quantiles, one constant per block, constants stored in 8 bits under a
// coarser level) and the capability page "Qlora 4 Bit Quantization With Nf4
// Fp4 Data Types And Lora Adapters", NF4 entry (block-wise absmax scaling).
//
// Layout: one workgroup per group of 256 consecutive blocks (blocks of 64,
// 128 or 256 elements: 64, 128 or 256 KB of W), with 4, 8 or 16 waves.
// Each wave walks 16 KB of the group, 256 elements per load instruction
// (1 KB of contiguous W):
// each lane owns four consecutive elements, and the 16, 32 or 64 lanes of a
// block reduce its absmax by butterfly shuffles.  Codes are packed in
// 64-element units whatever the block size.  4-bit codes are
// stored by every lane (128 contiguous bytes per instruction); 3- and 2-bit
// codes are ORed into their half block's words across the eight lanes of
// the half and stored by its first lane.  The kernel is bound by HBM (4 B
// read and at most 0.52 B written per weight).
#include "kernels.hpp"

namespace qn {

// The code of x in [-1, 1] is code_of_count(#{thresholds below x}).  The
// count comes from a bucket table instead of one compare per threshold:
// buckets split [-1, 1] by sign, binary exponent (2^-6 .. 2^0) and the top 4
// mantissa bits, with one bucket per sign for |x| < 2^-6 (1 + 1/16).  A
// bucket is at most 1/32 wide while consecutive thresholds of every code
// type are at least 0.08 apart, so it holds at most one threshold: the
// count is the bucket's base (thresholds below the whole bucket) plus
// (x > the threshold inside it, +inf if none).  A host test checks this
// against the direct count for every fp32 in [-1, 1].
constexpr int kBuckets = 224;  // 2 signs x 7 exponents x 16

// bucket[t] = {threshold inside (fp32 bits), base count}
template <class CT>
__device__ void build_buckets(uint2* bucket) {
  for (int t = threadIdx.x; t < kBuckets; t += blockDim.x) {
    const int sg = t / 112, ke = (t % 112) / 16, j = t % 16;
    const float lo = (ke == 0 && j == 0) ? 0.0f : ldexpf(1.0f + j / 16.0f, ke - 6);
    const float hi = ldexpf(1.0f + (j + 1) / 16.0f, ke - 6);
    uint32_t base = 0;
    float inside = __builtin_inff();
    for (int i = 0; i < CT::table.ndist - 1; ++i) {
      const float T = __builtin_bit_cast(float, CT::table.thr[i]);
      if (sg == 0) {  // x in [lo, hi)
        if (T < lo) ++base;
        else if (T < hi) inside = T;
      } else {        // x in (-hi, -lo]
        if (T <= -hi) ++base;
        else if (T <= -lo) inside = T;
      }
    }
    bucket[t] = make_uint2(__builtin_bit_cast(uint32_t, inside), base);
  }
}

template <class CT>
__device__ __forceinline__ uint32_t quant_code(float x, const uint2* bucket) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const int e = (int)((u >> 23) & 0xffu);
  const int sg = (int)(u >> 31);
  const int key = e < 121 ? sg * 112 : sg * 112 + (e - 121) * 16 + (int)((u >> 19) & 15u);
  const uint2 bk = bucket[key];
  const uint32_t n = bk.y + (x > __builtin_bit_cast(float, bk.x) ? 1u : 0u);
  return CT::code_of_count(n);
}

// fl32(a / b) from r = fl32(1 / b): q = fl32(a r) is within two ulps of
// a / b, the residual e = a - b q comes out of the fused multiply-add with at
// most a 2^-24 relative error, and one correction step q + e r lands within
// one ulp of the IEEE quotient (a division refinement in Markstein's form).
// Used for blocks with 2^-60 <= b <= 2^126 and |a| <= b, where every
// intermediate near a threshold is a normal number: the outcome then depends
// only on the mantissas, and a host test checks every divisor mantissa with
// every dividend whose quotient lies within 4 ulps of any threshold of any
// code type: the refined quotient is the IEEE one there, so every code is
// the one the IEEE quotient gives.  Other blocks take the IEEE division.
__device__ __forceinline__ float div_refined(float a, float b, float r) {
#pragma clang fp contract(off)
  const float q = a * r;
  const float e = __builtin_fmaf(-q, b, a);
  return __builtin_fmaf(e, r, q);
}

// Block size 64 << BS (BS = 0, 1, 2: 64, 128, 256 elements per constant).
// Code of x under a caller's codebook: the count of thresholds below x,
// one compare per threshold (they may lie arbitrarily close together, so
// the bucket table does not apply), mapped to the lowest code of that value.
__device__ __forceinline__ uint32_t user_code(float x, const UserTable& u) {
  uint32_t n = 0;
#pragma unroll
  for (int i = 0; i < 15; ++i) n += (x > u.thr[i]) ? 1u : 0u;
  const uint64_t map = ((uint64_t)u.code_hi << 32) | u.code_lo;
  return (uint32_t)(map >> (4 * n)) & 15u;
}

template <class CT>
__device__ __forceinline__ uint32_t zero_code() {
  if constexpr (CT::kUser) return 0u;  // not reached: user blocks take user_code
  else return CT::table.zero_code;
}

// 256 << BS threads (4 << BS waves): every wave walks 16 instructions of
// 256 elements whatever the block size, so larger blocks get more waves per
// group instead of longer walks.
template <class CT, int BS>
__global__ __launch_bounds__(256 << BS) void k_nf4_quantize(const float* __restrict__ W,
                                                      int64_t nblocks,
                                                      uint8_t* __restrict__ codes,
                                                      uint8_t* __restrict__ q8,
                                                      float* __restrict__ step, UserTable ut) {
  constexpr int kLanesPerBlock = 16 << BS;  // four elements per lane
  __shared__ float cabs[256];
  __shared__ float wmax[4];
  __shared__ uint2 bucket[kBuckets];
  if constexpr (!CT::kUser) {
    build_buckets<CT>(bucket);
    __syncthreads();
  }
  const int64_t g = blockIdx.x;
  const int64_t b0 = g * 256;  // first block of the group
  const int nb = (int)((nblocks - b0) < 256 ? (nblocks - b0) : 256);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int sub = lane & 15;  // lane within its 64-element unit: elements 4*sub .. 4*sub+3

  // Wave w walks elements 4096 w .. 4096 w + 4095 of the group, 256
  // elements (a 64-lane instruction of 16 bytes each) per iteration.
  for (int it = 0; it < 16; ++it) {
    const int64_t e0 = ((int64_t)(wave << 4) + it) * 256 + 4 * lane;  // element in group
    const int bi = (int)(e0 >> (6 + BS));                                    // block in group
    if (bi < nb) {
      const int64_t e = (b0 << (6 + BS)) + e0;  // element index in W
      const int64_t u = e >> 6;                 // its 64-element packing unit
      const f32x4 v = *reinterpret_cast<const f32x4*>(W + e);
      float m = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
#pragma unroll
      for (int off = kLanesPerBlock / 2; off >= 1; off >>= 1)
        m = fmaxf(m, __shfl_xor(m, off, kLanesPerBlock));
      uint32_t c0, c1, c2, c3;
      if constexpr (CT::kUser) {
        // IEEE-correct division for every block (the refined quotient is
        // checked only near the built-in thresholds); x = 0 in an all-zero
        // block, which then takes the code of the value nearest to zero
        c0 = user_code(m > 0.0f ? v[0] / m : 0.0f, ut);
        c1 = user_code(m > 0.0f ? v[1] / m : 0.0f, ut);
        c2 = user_code(m > 0.0f ? v[2] / m : 0.0f, ut);
        c3 = user_code(m > 0.0f ? v[3] / m : 0.0f, ut);
      } else if (m >= 0x1p-60f && m <= 0x1p126f) {
        const float r = 1.0f / m;  // IEEE-correct fp32 division
        c0 = quant_code<CT>(div_refined(v[0], m, r), bucket);
        c1 = quant_code<CT>(div_refined(v[1], m, r), bucket);
        c2 = quant_code<CT>(div_refined(v[2], m, r), bucket);
        c3 = quant_code<CT>(div_refined(v[3], m, r), bucket);
      } else if (m > 0.0f) {
        // tiny or huge block: IEEE-correct fp32 division (the compiler's default)
        c0 = quant_code<CT>(v[0] / m, bucket);
        c1 = quant_code<CT>(v[1] / m, bucket);
        c2 = quant_code<CT>(v[2] / m, bucket);
        c3 = quant_code<CT>(v[3] / m, bucket);
      } else {
        c0 = c1 = c2 = c3 = zero_code<CT>();  // all-zero block: the zero level
      }
      if constexpr (CT::kBits == 4) {
        const uint16_t packed = (uint16_t)(c0 | (c1 << 4) | (c2 << 8) | (c3 << 12));
        *reinterpret_cast<uint16_t*>(codes + u * 32 + sub * 2) = packed;
      } else {
        // elements 4 sub + t = 32 h + 8 g + 2 i + p of the unit
        const int h = sub >> 3, g = (sub >> 1) & 3, i0 = 2 * (sub & 1);
        const uint32_t cc[4] = {c0, c1, c2, c3};
        uint32_t wv[3] = {0u, 0u, 0u};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int i = i0 + (t >> 1), pp = t & 1;
          wv[pp] |= (cc[t] & 3u) << (8 * i + 2 * g);
          if (CT::kBits == 3) wv[2] |= ((cc[t] >> 2) & 1u) << ((8 * i + 2 + 2 * g + pp) & 31);
        }
#pragma unroll
        for (int j = 0; j < CT::kBits; ++j) {
          wv[j] |= __shfl_xor(wv[j], 1, 16);
          wv[j] |= __shfl_xor(wv[j], 2, 16);
          wv[j] |= __shfl_xor(wv[j], 4, 16);
        }
        if ((sub & 7) == 0) {
          uint32_t* dst =
              reinterpret_cast<uint32_t*>(codes + u * block_bytes<CT>() + h * half_bytes<CT>());
#pragma unroll
          for (int j = 0; j < CT::kBits; ++j) dst[j] = wv[j];
        }
      }
      if ((lane & (kLanesPerBlock - 1)) == 0) cabs[bi] = m;
    }
  }
  __syncthreads();

  // Double quantization of this group's constants, by the first four
  // waves (one thread per block); the others hold c = 0.
  const int t = threadIdx.x;
  float c = (t < nb) ? cabs[t] : 0.0f;
  float m = c;
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  if (lane == 0 && wave < 4) wmax[wave] = m;
  __syncthreads();
  const float smax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const float st = smax / 255.0f;
  if (t < nb) {
    uint32_t q = 0;
    if (st > 0.0f) {
      const float r = __builtin_rintf(c / st);  // round half to even
      q = (r >= 255.0f) ? 255u : (uint32_t)r;
    }
    q8[b0 + t] = (uint8_t)q;
  }
  if (t == 0) step[g] = st;
}

// Standalone dequantizer: w = bf16_rne(value[code] * fl32(q8 * step)).
// Each thread expands eight codes (eight weights) into 16 bytes of bf16.
template <class CT>
__global__ __launch_bounds__(256) void k_nf4_dequantize(const uint8_t* __restrict__ codes,
                                                        const uint8_t* __restrict__ q8,
                                                        const float* __restrict__ step,
                                                        int64_t n8, int bshift,
                                                        uint16_t* __restrict__ out,
                                                        UserTable ut) {
  __shared__ float lv[16];
  if (threadIdx.x < 16) lv[threadIdx.x] = level_of<CT>(ut, threadIdx.x);
  __syncthreads();
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n8;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t b = i >> 3;  // 8 groups of 8 weights per 64-element block
    uint32_t w;
    if constexpr (CT::kBits == 4) {
      w = *reinterpret_cast<const uint32_t*>(codes + i * 4);
    } else {
      const int hh = (int)((i >> 2) & 1), g = (int)(i & 3);
      w = nibbles<CT>(load_half<CT>(codes + b * block_bytes<CT>() + hh * half_bytes<CT>()), g);
    }
    const int64_t cb = b >> bshift;  // the block of 64 << bshift elements
    const float chat = (float)q8[cb] * step[cb >> 8];
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float lo = lv[(w >> (8 * j)) & 15u] * chat;
      const float hi = lv[(w >> (8 * j + 4)) & 15u] * chat;
      o[j] = pack_bf16x2(lo, hi);
    }
    *reinterpret_cast<u32x4*>(out + i * 8) = o;
  }
}

hipError_t launch_nf4_quantize(const float* W, int64_t nblocks, uint8_t* codes, uint8_t* q8,
                               float* step, int code, int bshift, const UserTable* ut,
                               hipStream_t stream) {
  const int64_t ngroups = (nblocks + 255) / 256;
  const UserTable u = ut ? *ut : UserTable{};
  return with_any_code(code, [&](auto ct) {
    using CT = decltype(ct);
    if (bshift == 2)
      hipLaunchKernelGGL((k_nf4_quantize<CT, 2>), dim3((unsigned)ngroups), dim3(1024), 0, stream,
                         W, nblocks, codes, q8, step, u);
    else if (bshift == 1)
      hipLaunchKernelGGL((k_nf4_quantize<CT, 1>), dim3((unsigned)ngroups), dim3(512), 0, stream,
                         W, nblocks, codes, q8, step, u);
    else
      hipLaunchKernelGGL((k_nf4_quantize<CT, 0>), dim3((unsigned)ngroups), dim3(256), 0, stream,
                         W, nblocks, codes, q8, step, u);
    return hipGetLastError();
  });
}

hipError_t launch_nf4_dequantize(const uint8_t* codes, const uint8_t* q8, const float* step,
                                 int64_t nelem, uint16_t* out, int code, int bshift,
                                 const UserTable* ut, hipStream_t stream) {
  const int64_t n8 = nelem / 8;
  int64_t grid = (n8 + 255) / 256;
  if (grid > 65536) grid = 65536;
  const UserTable u = ut ? *ut : UserTable{};
  return with_any_code(code, [&](auto ct) {
    hipLaunchKernelGGL(k_nf4_dequantize<decltype(ct)>, dim3((unsigned)grid), dim3(256), 0, stream,
                       codes, q8, step, n8, bshift, out, u);
    return hipGetLastError();
  });
}

}  // namespace qn
