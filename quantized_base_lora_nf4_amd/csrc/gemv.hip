// Forward pass for few tokens (M <= 16): the whole cost is streaming the
// packed 4-bit weight (codes + 8-bit constants + fp32 steps, 4.13 bits per
// weight) out of HBM once, so the kernel is shaped for bandwidth, not for
// MFMA throughput.
//
// Dequantize-on-the-fly as in "QLoRA: fine-tuning a 65B model on one GPU",
// section "Where the memory goes".  A memory-bound stream leaves only a few
// lane operations per weight, so the codes are expanded to *unscaled* bf16
// levels (a 256-entry byte table in LDS, one lookup per code byte), the
// MFMA sums one 64-element block at a time, and the block constant
// fl32(q8 * step) multiplies that block's fp32 partial sum.  The result
// differs from using the bf16-rounded dequantized weight only by the bf16
// rounding of the levels (relative 2^-9 per weight); accumulation is fp32.
//
// Two launches per call:
//  1. k_lora_down_part: fp32 partial sums of U = X A^T over S slices of K.
//  2. k_qgemv: Y = X W^T + s U B^T.  A workgroup owns 16 G weight rows and
//     all of K; its KW waves each take a contiguous range of K, and their
//     partial sums are added in LDS.  The epilogue sums the U partials,
//     adds the LoRA term and stores bf16 Y (and bf16 U when asked for).
//
// Operand layout (MFMA 16x16x32 bf16, A = X rows, B = weight rows, so that
// the four results of a lane share one weight row and one block constant):
// per double step (blocks kb, kb+1) lane l loads 16 bytes of weight row
// l % 16 at byte 32 kb + 16 (l / 16), i.e. lanes 0-31 hold block kb and
// lanes 32-63 block kb+1.  One cross-half swap of two code words
// (v_permlane32_swap) leaves every lane with two 8-code words of each
// block, so each MFMA contracts codes of a single block.  Word j of lane
// group q then holds codes 32 (q & 1) + 16 (q >> 1) + 8 (j & 1) .. +7 of
// block kb + (j >> 1); the X fragment of MFMA j uses the same positions.
#include "kernels.hpp"

namespace qn {

namespace {

// Eight codes -> four packed bf16 level pairs, by a byte-indexed LDS table.
// The table is replicated 16 times, entry b of copy l at word 16 b + l, and
// lane l reads copy l % 16 (lutl = table + l % 16): the 16 lanes that the
// LDS serves together then always hit 16 different banks, whatever the codes
// (random indices into a single copy stall the LDS on bank conflicts).
__device__ __forceinline__ u32x4 levels8_lut(uint32_t w, const uint32_t* lutl) {
  return u32x4{lutl[16 * (w & 0xffu)], lutl[16 * ((w >> 8) & 0xffu)],
               lutl[16 * ((w >> 16) & 0xffu)], lutl[16 * (w >> 24)]};
}
constexpr int kLutWords = 256 * 16;

// ---------------------------------------------------------------------------
// U partial sums: part[s][m][j] = sum over k in slice s of X[m][k] A[j][k].
// Grid (S, ceil(r / 64)); wave w of a workgroup owns adapter rows
// 64 blockIdx.y + 16 w .. +15.  MFMA 16x16x32: A = X rows, B = A rows.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_lora_down_part(const uint16_t* __restrict__ X, int64_t M,
                                                        const uint16_t* __restrict__ A, int32_t r,
                                                        int64_t K, int64_t slice,
                                                        float* __restrict__ part) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i16 = lane & 15, q = lane >> 4;
  const int64_t j = (int64_t)blockIdx.y * 64 + wave * 16 + i16;
  const bool mvalid = i16 < M, jvalid = j < r;
  const int64_t k0 = (int64_t)blockIdx.x * slice;
  int64_t k1 = k0 + slice;
  if (k1 > K) k1 = K;
  const uint16_t* xr = X + (mvalid ? i16 : 0) * K + 8 * q;
  const uint16_t* ar = A + (jvalid ? j : 0) * K + 8 * q;
  const u32x4 zero = u32x4{0u, 0u, 0u, 0u};
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  // Batches of 8 steps: all 16 loads of a batch are issued (unconditionally:
  // invalid rows re-read row 0 and are zeroed after) before the first use,
  // so a batch costs one memory latency instead of eight.
  constexpr int U = 8;
  int64_t k = k0;
  for (; k + 32 * U <= k1; k += 32 * U) {
    u32x4 xa[U], aa[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      xa[u] = *reinterpret_cast<const u32x4*>(xr + k + 32 * u);
      aa[u] = *reinterpret_cast<const u32x4*>(ar + k + 32 * u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      acc = mfma16(as_bf16x8(mvalid ? xa[u] : zero), as_bf16x8(jvalid ? aa[u] : zero), acc);
  }
  for (; k < k1; k += 32) {
    const u32x4 xa = *reinterpret_cast<const u32x4*>(xr + k);
    const u32x4 aa = *reinterpret_cast<const u32x4*>(ar + k);
    acc = mfma16(as_bf16x8(mvalid ? xa : zero), as_bf16x8(jvalid ? aa : zero), acc);
  }
  // D[m = 4 q + v][j]
  float* out = part + (int64_t)blockIdx.x * M * r;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int m = 4 * q + v;
    if (m < M && jvalid) out[m * r + j] = acc[v];
  }
}

struct GemvArgs {
  const uint8_t* codes;
  const uint8_t* q8;
  const float* step;
  const uint16_t* X;
  int64_t M, N, K;
  const float* upart;  // [us][M][r]
  int32_t us;
  const uint16_t* B;
  int32_t r;
  float s;
  uint16_t* Y;
  uint16_t* U_out;  // nullable, bf16 [M][r]
};

#ifndef QN_GEMV_PD
#define QN_GEMV_PD 3
#endif

// Dynamic LDS of k_qgemv, in 4-byte words: the byte table (kLutWords), the U sums
// (M r), then a region holding the block constants of the workgroup's rows
// during the main loop (16 G rows of odd stride kblocks | 1, so that the 16
// rows a wave reads at once sit in 16 different banks) and the waves'
// partial sums after it (KW G 256).
__host__ __device__ constexpr int64_t gemv_lds_words(int G, int KW, int64_t M, int64_t r,
                                                     int64_t kblocks) {
  const int64_t chat = 16 * G * (kblocks | 1), red = (int64_t)KW * G * 256;
  return kLutWords + M * r + (chat > red ? chat : red);
}

template <int G, int KW, int PD, class CT>
__global__ __launch_bounds__(64 * KW) void k_qgemv(GemvArgs p) {
  constexpr int NT = 64 * KW;
  extern __shared__ float lds[];
  uint32_t* lut = reinterpret_cast<uint32_t*>(lds);
  float* ush = lds + kLutWords;
  float* chat_t = ush + p.M * p.r;  // [16 G][kblocks | 1] during the main loop
  float* red = chat_t;              // [KW][G][4][64] after it

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i16 = lane & 15, q = lane >> 4;
  const int64_t M = p.M, N = p.N, K = p.K;
  const int64_t kblocks = K >> 6;
  const int64_t kbs = kblocks | 1;  // row stride of the constant table
  const int64_t n0 = (int64_t)blockIdx.x * 16 * G;

  // Full double steps [d0, d1) of this wave, out of T = kblocks / 2; an odd
  // last block is a separate tail step of the last wave.
  const int64_t T = kblocks >> 1;
  const int64_t d0 = T * wave / KW, d1 = T * (wave + 1) / KW;
  const bool odd_tail = (kblocks & 1) && wave == KW - 1;

  // Lane quarter q reads half (q & 1) of block (q >> 1) of each double step.
  const uint8_t* crow[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    int64_t n = n0 + 16 * g + i16;
    if (n >= N) n = N - 1;  // computed and dropped
    crow[g] = p.codes + n * kblocks * block_bytes<CT>() + (q >> 1) * block_bytes<CT>() +
              (q & 1) * half_bytes<CT>();
  }
  // X fragment of word j: row i16, columns 64 (kb + (j >> 1)) + xo + 8 (j & 1).
  // Rows past M re-read row 0; their results are never stored.
  const int xo = 32 * (q & 1) + 16 * (q >> 1);
  const uint16_t* xrow = p.X + (i16 < M ? i16 : 0) * K + xo;
  // this lane's rows of the block-constant table
  const float* crow_t[G];
#pragma unroll
  for (int g = 0; g < G; ++g) crow_t[g] = chat_t + (16 * g + i16) * kbs;

  // Raw loads of one double step (codes, X fragments).  Nothing is computed
  // from them at issue, so issuing never waits for a load.
  struct Slot {
    HalfRaw<CT::kBits> c[G];
    u32x4 x[4];
  };
  Slot sl[PD];

  // Every call issues the same loads (no branches), so that the compiler can
  // count them and wait only for the step being consumed.  Steps past the
  // end re-read the last one.  The tail form covers the single block kb:
  // lanes 32-63 re-read it (its second half gets constant 0).
  auto issue = [&](Slot& S, int64_t d, bool tail) {
    if (d >= d1 && !tail) d = d1 - 1;
    const int64_t kb = 2 * d;
    const int64_t off = ((tail && q >= 2) ? kb - 1 : kb) * block_bytes<CT>();
    const int64_t kb2 = tail ? kb : kb + 1;
#pragma unroll
    for (int g = 0; g < G; ++g) S.c[g] = load_half<CT>(crow[g] + off);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      S.x[j] = *reinterpret_cast<const u32x4*>(xrow + 64 * ((j >> 1) ? kb2 : kb) + 8 * (j & 1));
  };

  f32x4 acc[G];
#pragma unroll
  for (int g = 0; g < G; ++g) acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const Slot& S, int64_t d, bool tail) {
    const int64_t kb = 2 * d;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      u32x4 c;
#pragma unroll
      for (int j = 0; j < 4; ++j) c[j] = nibbles<CT>(S.c[g], j);
      // lanes 0-31: (block kb words 0, 1 | words 2, 3) -> keep 0, 1, take the
      // other half's 0, 1 into 2, 3; lanes 32-63 the mirror image.
      const auto s02 = __builtin_amdgcn_permlane32_swap(c[0], c[2], false, false);
      const auto s13 = __builtin_amdgcn_permlane32_swap(c[1], c[3], false, false);
      c[0] = s02[0];
      c[2] = s02[1];
      c[1] = s13[0];
      c[3] = s13[1];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const u32x4 w0 = levels8_lut(c[2 * h], lut + i16);
        const u32x4 w1 = levels8_lut(c[2 * h + 1], lut + i16);
        f32x4 pb = mfma16(as_bf16x8(S.x[2 * h]), as_bf16x8(w0), f32x4{0.f, 0.f, 0.f, 0.f});
        pb = mfma16(as_bf16x8(S.x[2 * h + 1]), as_bf16x8(w1), pb);
        const float chat = (h && tail) ? 0.0f : crow_t[g][kb + h];
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[g][v] += chat * pb[v];
      }
    }
  };

  const bool active = d0 < d1;  // the wave has full steps (uniform)
  if (active) {
#pragma unroll
    for (int u = 0; u < PD - 1; ++u) issue(sl[u], d0 + u, false);
  }
  // Prologue, overlapping the first loads: the byte table, the block
  // constants fl32(q8 * step) of rows n0 .. n0 + 16 G - 1, and the U sums of
  // the partial slices written by the previous launch on this stream.  All
  // of a thread's loads are issued before any is used (one latency).
  for (int e = tid; e < kLutWords; e += NT) {
    const int b = e >> 4;  // copy e % 16 of entry b
    lut[e] = pack_bf16x2(code_value<CT>(b & 15), code_value<CT>(b >> 4));
  }
  {
    // The workgroup's constants are the contiguous q8 range starting at
    // n0 kblocks (a multiple of 16 bytes), 16 G kblocks bytes long; rows
    // past N read clamped bytes (their results are dropped).
    const int64_t qtot = N * kblocks, qbase = n0 * kblocks;
    const int64_t nchunk = (16 * G * kblocks + 15) / 16;
    for (int64_t c = tid; c < nchunk; c += NT) {
      const int64_t o = qbase + 16 * c;
      u32x4 qv;
      if (o + 16 <= qtot) {
        qv = *reinterpret_cast<const u32x4*>(p.q8 + o);
      } else {
        uint32_t b[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) b[i] = p.q8[o + i < qtot ? o + i : qtot - 1];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          qv[i] = b[4 * i] | (b[4 * i + 1] << 8) | (b[4 * i + 2] << 16) | (b[4 * i + 3] << 24);
      }
      const int64_t ng = (qtot + 255) >> 8;
      const int64_t g0 = o >> 8 < ng ? o >> 8 : ng - 1;
      const int64_t g1 = (o + 15) >> 8 < ng ? (o + 15) >> 8 : ng - 1;
      const float st0 = p.step[g0], st1 = p.step[g1];
      const int64_t split = (g0 + 1) << 8;  // first block of group g0 + 1
      float cv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i)
        cv[i] = (float)((qv[i >> 2] >> (8 * (i & 3))) & 0xffu) * (o + i < split ? st0 : st1);
      // element 16 c + i is block kb of table row `row`
      int64_t row = (16 * c) / kblocks, kb = 16 * c - row * kblocks;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (row < 16 * G) chat_t[row * kbs + kb] = cv[i];
        if (++kb == kblocks) {
          kb = 0;
          ++row;
        }
      }
    }
  }
  {
    const int64_t ur = (int64_t)M * p.r;
    // slices in order, eight loads in flight at a time
    constexpr int kBatch = 8;
    for (int64_t e = tid; e < ur; e += NT) {
      float u = 0.0f;
      for (int sp0 = 0; sp0 < p.us; sp0 += kBatch) {
        float v[kBatch];
#pragma unroll
        for (int i = 0; i < kBatch; ++i)
          v[i] = p.upart[(int64_t)(sp0 + i < p.us ? sp0 + i : sp0) * ur + e];
#pragma unroll
        for (int i = 0; i < kBatch; ++i)
          if (sp0 + i < p.us) u += v[i];
      }
      ush[e] = u;
    }
  }
  __syncthreads();

  // A ring of PD register slots keeps PD - 1 steps of loads in flight while
  // a step is consumed.  Loads are counted in issue order, so codes and X
  // fragments travel in the same slot, and the scheduling barriers keep each
  // step's loads ahead of the arithmetic of the step before it: the wait
  // before a step then covers that step's own loads only.
  int64_t d = d0;
  for (; d + PD <= d1; d += PD) {  // slots 0 .. PD-2 hold steps d .. d+PD-2 on entry
#pragma unroll
    for (int u = 0; u < PD; ++u) {
      issue(sl[(u + PD - 1) % PD], d + u + PD - 1, false);
      __builtin_amdgcn_sched_barrier(0);
      compute(sl[u], d + u, false);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int u = 0; u < PD - 1; ++u)
    if (d + u < d1) compute(sl[u], d + u, false);
  if (odd_tail) {
    issue(sl[PD - 1], T, true);
    compute(sl[PD - 1], T, true);
  }
  __syncthreads();  // the constant table becomes the reduction buffer

#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int v = 0; v < 4; ++v) red[((wave * G + g) * 4 + v) * 64 + lane] = acc[g][v];
  __syncthreads();

  for (int o = tid; o < G * 4 * 64; o += NT) {
    const int l = o & 63, v = (o >> 6) & 3, g = o >> 8;
    float y = 0.0f;
#pragma unroll
    for (int w = 0; w < KW; ++w) y += red[((w * G + g) * 4 + v) * 64 + l];
    const int64_t m = 4 * (l >> 4) + v, n = n0 + 16 * g + (l & 15);
    if (m < M && n < N) {
      float lora = 0.0f;
      const uint16_t* brw = p.B + n * p.r;
      for (int j = 0; j < p.r; ++j) lora += ush[m * p.r + j] * bf16_to_f32(brw[j]);
      p.Y[m * N + n] = f32_to_bf16(y + p.s * lora);
    }
  }
  if (p.U_out && blockIdx.x == 0) {
    for (int64_t e = tid; e < (int64_t)M * p.r; e += NT) p.U_out[e] = f32_to_bf16(ush[e]);
  }
}

}  // namespace

bool gemv_fits(int64_t M, int32_t r, int64_t K) {
  // the workgroup's LDS within 96 KB (K up to about 32000 at 16 tokens and rank 256)
  return M <= kGemvMaxM && 4 * gemv_lds_words(2, 8, M, r, K / 64) <= 96 * 1024;
}

int gemv_lora_slices(int64_t M, int32_t r, int64_t K) {
  // Slices of at least 256 columns (one batch of loads per wave), at most
  // 32, and at most 8192 partial values in all: k_qgemv's prologue sums
  // them, M r values per slice.
  int64_t s = K / 256;
  if (s > 32) s = 32;
  while (s > 1 && s * M * r > 8192) s /= 2;
  if (s < 1) s = 1;
  return (int)s;
}

size_t gemv_workspace_bytes(int64_t M, int32_t r, int64_t K) {
  return (size_t)gemv_lora_slices(M, r, K) * M * r * sizeof(float);
}

template <int G>
hipError_t launch_qgemv_g(const GemvArgs& a, int code, hipStream_t stream) {
  constexpr int KW = 8, PD = QN_GEMV_PD;
  static const hipError_t attr = [] {
    // dynamic LDS above the default 64 KB needs the limit raised, once per
    // instantiation
    hipError_t r = hipSuccess;
    for (int id = 0; id < 4; ++id) {
      const hipError_t e = with_code(id, [](auto ct) {
        return hipFuncSetAttribute(
            reinterpret_cast<const void*>(&k_qgemv<G, KW, PD, decltype(ct)>),
            hipFuncAttributeMaxDynamicSharedMemorySize, 96 * 1024);
      });
      if (r == hipSuccess) r = e;
    }
    return r;
  }();
  if (attr != hipSuccess) return attr;
  const size_t lds = 4 * (size_t)gemv_lds_words(G, KW, a.M, a.r, a.K / 64);
  const dim3 grid((unsigned)((a.N + 16 * G - 1) / (16 * G)));
  with_code(code, [&](auto ct) {
    hipLaunchKernelGGL((k_qgemv<G, KW, PD, decltype(ct)>), grid, dim3(64 * KW), lds,
                       stream, a);
    return 0;
  });
  return hipGetLastError();
}

hipError_t launch_qgemv(const Nf4View& w, const uint16_t* X, int64_t M, const uint16_t* A,
                        const uint16_t* B, int32_t r, float s, uint16_t* Y, uint16_t* U_out,
                        float* upart, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  const int us = gemv_lora_slices(M, r, w.K);
  const int64_t slice = (w.K / us + 31) / 32 * 32;
  dim3 gu((unsigned)((w.K + slice - 1) / slice), (unsigned)((r + 63) / 64));
  hipLaunchKernelGGL(k_lora_down_part, gu, dim3(256), 0, stream, X, M, A, r, w.K, slice, upart);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ev0 && (e = hipEventRecord(ev0, stream)) != hipSuccess) return e;
  const GemvArgs a{w.codes, w.q8, w.step, X, M, w.N, w.K, upart, (int32_t)gu.x, B, r, s, Y, U_out};
  const int64_t kblocks = w.K / 64;
  // 16 G weight rows per workgroup, K split over its 8 waves.
  //  - G = 7 when the 16-row groups make exactly one workgroup of 7 per CU
  //    (a 28672-row weight on 256 CUs): no CU gets more rows than another,
  //    and each CU loads the X fragments once.
  //  - G = 1 for one or two tokens when G = 2 would leave at most one
  //    workgroup (8 waves) per CU: twice the waves keep more loads in
  //    flight.  With more tokens the X fragments, loaded once per
  //    workgroup, cost more than that gains.
  //  - G = 2 otherwise.
  static const int cus = [] {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    return n;
  }();
  const int64_t groups = (w.N + 15) / 16;
  const bool g7 = cus > 0 && groups % (7 * (int64_t)cus) == 0 &&
                  4 * gemv_lds_words(7, 8, M, r, kblocks) <= 96 * 1024;
  const bool g1 = !g7 && M <= 2 && cus > 0 && groups <= 2 * (int64_t)cus;
  e = g7   ? launch_qgemv_g<7>(a, w.code, stream)
      : g1 ? launch_qgemv_g<1>(a, w.code, stream)
           : launch_qgemv_g<2>(a, w.code, stream);
  if (e != hipSuccess) return e;
  if (ev1) e = hipEventRecord(ev1, stream);
  return e;
}

}  // namespace qn
