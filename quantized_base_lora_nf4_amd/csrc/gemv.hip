// Forward pass for few tokens (M <= 16): the whole cost is streaming the
// packed 4-bit weight (codes + 8-bit constants + fp32 steps, 4.13 bits per
// weight) out of HBM once, so the kernel is shaped for bandwidth, not for
// MFMA throughput.
//
// Dequantize-on-the-fly as in "QLoRA: fine-tuning a 65B model on one GPU",
// section "Where the memory goes".  A memory-bound stream leaves only a few
// lane operations per weight, so the codes are expanded to *unscaled* bf16
// levels (a 256-entry byte table in LDS, one lookup per code byte), the
// MFMA sums one 64-element code block at a time, and the block constant
// fl32(q8 * step) (of the 64-, 128- or 256-element constant block it lies
// in) multiplies that block's fp32 partial sum.  The result
// differs from using the bf16-rounded dequantized weight only by the bf16
// rounding of the levels (relative 2^-9 per weight); accumulation is fp32.
//
// Two launches per call:
//  1. k_lora_down_part: fp32 partial sums of U = X A^T over S slices of K.
//  2. k_qgemv: Y = X W^T + s U B^T.  A workgroup owns 16 G weight rows and
//     all of K; its KW waves split K (wave pairs share a range and take its
//     even and odd double steps), and their partial sums are added in LDS.
//     With G = 7 each wave walks its steps in chunks, one row group after
//     another within a chunk; otherwise step by step over all groups.  The
//     epilogue sums the U partials, adds the LoRA term and stores bf16 Y
//     (and bf16 U when asked for).
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

// At most this many U partial slices (gemv_lora_slices).
constexpr int kGemvMaxSlices = 32;
// A per-lane buffer offset past every buffer this file reads through a
// buffer resource (each under 2^31 bytes): such a load returns 0.
constexpr int kPastEnd = INT32_MIN;

// ---------------------------------------------------------------------------
// U partial sums: part[m][j][s] (slices padded to kGemvMaxSlices, so that
// the slices of one sum are one contiguous 128-byte row) = sum over k in
// slice s of X[m][k] A[j][k] for s < S, and 0 for the padding slices.
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
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int m = 4 * q + v;
    if (m < M && jvalid) part[(m * r + j) * kGemvMaxSlices + blockIdx.x] = acc[v];
  }
  // the slices past the grid read as zeros, so that a sum may take all of
  // them in order
  if (blockIdx.x == 0) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = 4 * q + v;
      if (m < M && jvalid)
        for (int s = gridDim.x; s < kGemvMaxSlices; ++s)
          part[(m * r + j) * kGemvMaxSlices + s] = 0.0f;
    }
  }
}

struct GemvArgs {
  const uint8_t* codes;
  const uint8_t* q8;
  const float* step;
  const uint16_t* X;
  int64_t M, N, K;
  const float* upart;  // [M][r][kGemvMaxSlices]: the slices, then zeros
  const uint16_t* B;
  int32_t r;
  float s;
  uint16_t* Y;
  uint16_t* U_out;  // nullable, bf16 [M][r]
  int bshift;       // block size 64 << bshift
  UserTable ut;     // the caller's codebook (CodeUser types only)
};

#ifndef QN_GEMV_PD
#define QN_GEMV_PD 3
#endif

// Dynamic LDS of k_qgemv, in 4-byte words: the byte table (kLutWords), the U sums
// (M r), then a region holding the block constants of the workgroup's rows
// during the main loop (16 G rows of odd stride kblocks | 1, so that the 16
// rows a wave reads at once sit in 16 different banks) and the waves'
// partial sums after it (KW G 256); with seven groups, the workgroup's
// adapter rows last, 16-byte aligned.
__host__ __device__ constexpr int64_t gemv_b_words(int G, int64_t r) {
  // 16 G x r bf16 in whole KB (one direct-to-LDS copy instruction each)
  return G == 7 ? (16 * G * r * 2 + 1023) / 1024 * 256 : 0;
}
__host__ __device__ constexpr int64_t gemv_lds_words(int G, int KW, int64_t M, int64_t r,
                                                     int64_t kblocks) {
  const int64_t chat = 16 * G * (kblocks | 1), red = (int64_t)KW * G * 256;
  const int64_t base = kLutWords + M * r + (chat > red ? chat : red);
  return G == 7 ? ((base + 3) & ~(int64_t)3) + gemv_b_words(G, r) : base;
}

// One row group runs two workgroups per CU (16 waves): the register budget
// is held to 128 so that both fit.
template <int G, int KW, int PD, class CT>
__global__ __launch_bounds__(64 * KW) __attribute__((amdgpu_waves_per_eu(G == 1 ? 4 : 1)))
void k_qgemv(GemvArgs p) {
  constexpr int NT = 64 * KW;
  extern __shared__ float lds[];
  uint32_t* lut = reinterpret_cast<uint32_t*>(lds);
  float* ush = lds + kLutWords;
  float* chat_t = ush + p.M * p.r;  // [16 G][kblocks | 1] during the main loop
  float* red = chat_t;              // [KW][G][4][64] after it
  // G = 7: the workgroup's adapter rows, copied in by the prologue (bf16 [16 G][r])
  const int64_t chat_words = 16 * G * ((p.K >> 6) | 1), red_words = (int64_t)KW * G * 256;
  const int64_t cr_words = chat_words > red_words ? chat_words : red_words;
  uint16_t* bsh = reinterpret_cast<uint16_t*>(lds + ((kLutWords + p.M * p.r + cr_words + 3) & ~3));

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i16 = lane & 15, q = lane >> 4;
  // seven row groups: row-group-major main loop (below)
  constexpr bool kRowMajor = G == 7;
  const int64_t M = p.M, N = p.N, K = p.K;
  const int64_t kblocks = K >> 6;
  const int64_t kbs = kblocks | 1;  // row stride of the constant table
  const int64_t n0 = (int64_t)blockIdx.x * 16 * G;

  // Double steps (two blocks, 64 code bytes of a row at 4 bits) out of
  // T = kblocks / 2; an odd last block is a separate tail step of the last
  // wave.  Waves 2j and 2j + 1 share the range [e0, e1) and take its even
  // and odd steps: a step reads half of each row's 128-byte cache lines, so
  // the partner wave asks for the other half at about the same time.  With
  // contiguous ranges per wave the other half was requested a step later,
  // by which time many lines had left the L2 under the 16 G rows x 8 waves
  // of every workgroup: at 28672 x 8192 the kernel fetched 1.3-1.45 times
  // the weight bytes.  Local steps [d0, d1) of a wave are double steps
  // base + 2 d.
  const int64_t T = kblocks >> 1;
  const int64_t e0 = T * (wave >> 1) / (KW / 2), e1 = T * ((wave >> 1) + 1) / (KW / 2);
  const int64_t base = e0 + (wave & 1);
  const int64_t d0 = 0, d1 = e1 > base ? (e1 - base + 1) / 2 : 0;
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
    if (!tail) d = base + 2 * d;  // the tail step is double step T itself
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

  // One step as 2 G chains (group g, block h of the double step): table
  // lookups -> two MFMAs -> scaling by the block constant.  The chains are
  // software-pipelined: the lookups of chain c + 1 are issued before the
  // MFMAs of chain c and the scaling of chain c - 1, so the LDS latency of
  // a chain overlaps the work of its neighbours (one chain after another
  // left the wave waiting on the LDS once per chain).
  auto compute = [&](const Slot& S, int64_t d, bool tail) {
    if (!tail) d = base + 2 * d;
    const int64_t kb = 2 * d;
    constexpr int NC = 2 * G;
    u32x4 cw[G];  // per group: words 0, 1 of block kb and 2, 3 of block kb + 1
#pragma unroll
    for (int g = 0; g < G; ++g) {
      u32x4 c;
#pragma unroll
      for (int j = 0; j < 4; ++j) c[j] = nibbles<CT>(S.c[g], j);
      // lanes 0-31: (block kb words 0, 1 | words 2, 3) -> keep 0, 1, take the
      // other half's 0, 1 into 2, 3; lanes 32-63 the mirror image.  The
      // swap overwrites both operands: the copies keep it from tying up the
      // loaded registers (which made the compiler wait for loads still in
      // flight for later steps).
#pragma unroll
      for (int j = 0; j < 2; ++j) c[j] = __builtin_amdgcn_mov_dpp(c[j], 0xE4, 0xf, 0xf, false);
      const auto s02 = __builtin_amdgcn_permlane32_swap(c[0], c[2], false, false);
      const auto s13 = __builtin_amdgcn_permlane32_swap(c[1], c[3], false, false);
      cw[g] = u32x4{s02[0], s13[0], s02[1], s13[1]};
    }
    u32x4 wl[2][2];  // looked-up levels of two chains
    float ch[2];     // their block constants
    f32x4 pq[2];     // MFMA sums of two chains
    auto lookup = [&](int c) {
      const int g = c >> 1, h = c & 1;
      wl[c & 1][0] = levels8_lut(cw[g][2 * h], lut + i16);
      wl[c & 1][1] = levels8_lut(cw[g][2 * h + 1], lut + i16);
      ch[c & 1] = (h && tail) ? 0.0f : crow_t[g][kb + h];
    };
    auto mma = [&](int c) {
      const int h = c & 1;
      const f32x4 pb = mfma16(as_bf16x8(S.x[2 * h]), as_bf16x8(wl[c & 1][0]), f32x4{0.f, 0.f, 0.f, 0.f});
      pq[c & 1] = mfma16(as_bf16x8(S.x[2 * h + 1]), as_bf16x8(wl[c & 1][1]), pb);
    };
    auto scale = [&](int c) {
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[c >> 1][v] += ch[c & 1] * pq[c & 1][v];
    };
    lookup(0);
#pragma unroll
    for (int c = 0; c <= NC; ++c) {
      if (c >= 1) scale(c - 1);  // reads ch of chain c - 1 before lookup(c + 1) reuses it
      if (c + 1 < NC) lookup(c + 1);
      if (c < NC) mma(c);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  const bool active = d0 < d1;  // the wave has full steps (uniform)
  // With two or more row groups the first steps' loads go out behind the
  // prologue's own loads, so that the prologue waits for those (about one
  // latency) and not for the whole chip's first burst of weight codes
  // (4-5 % faster at 28672 x 8192, 2-4 % at 8192 x 8192 with G = 2).  With
  // one group (two workgroups per CU) issuing them first was faster
  // (17.5 against 20.0 us at 8192 x 8192).
  constexpr bool kLateFirst = G >= 2;
  // Row-group-major state (G = 7; unused otherwise): chunks of DW double
  // steps, one row group after another within a chunk (see the main loop).
  constexpr int DW = 4;
  typedef HalfRaw<CT::kBits> Codes[DW];
  u32x4 xf[DW][4];
  Codes cs[2];
  auto step_kb = [&](int64_t c, int j) {  // first block of local step DW c + j (clamped)
    int64_t dd = DW * c + j;
    if (dd >= d1) dd = d1 - 1;
    return 2 * (base + 2 * dd);
  };
  // Buffer loads: a per-lane 32-bit offset (the lane's row) plus the
  // step's offset, which is uniform, so no 64-bit address per load is
  // kept in vector registers (the codes are under 2 GiB by the C ABI, X
  // is at most 16 K bf16 rows of K).
  const __amdgpu_buffer_rsrc_t crs = bytes_rsrc(p.codes, N * kblocks * block_bytes<CT>());
  const __amdgpu_buffer_rsrc_t xrs = bytes_rsrc(p.X, 2 * M * K);
  int cvo[G];
#pragma unroll
  for (int g = 0; g < G; ++g) cvo[g] = (int)(crow[g] - p.codes);
  const int xvo = (int)(2 * (xrow - p.X));
  auto issue_x = [&](int64_t c) {
#pragma unroll
    for (int j = 0; j < DW; ++j) {
      const int kb = (int)step_kb(c, j);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        xf[j][i] = __builtin_amdgcn_raw_buffer_load_b128(
            xrs, xvo, 2 * (64 * (kb + (i >> 1)) + 8 * (i & 1)), 0);
    }
  };
  auto issue_c = [&](Codes& cd, int64_t c, int g) {
#pragma unroll
    for (int j = 0; j < DW; ++j)
      cd[j] = load_half<CT>(crs, cvo[g], (int)(step_kb(c, j) * block_bytes<CT>()));
  };
  auto issue_first = [&]() {
    if (active) {
      if constexpr (kRowMajor) {
        issue_c(cs[0], 0, 0);  // the first group's codes of the first chunk
      } else {
#pragma unroll
        for (int u = 0; u < PD - 1; ++u) issue(sl[u], d0 + u, false);
      }
    }
  };
  if constexpr (!kLateFirst) issue_first();
  // Prologue, overlapping the first loads: the U sums of the partial slices
  // written by the previous launch on this stream, the block constants
  // fl32(q8 * step) of rows n0 .. n0 + 16 G - 1, and the byte table.  The
  // loads go through buffer resources (an offset past the end reads 0), so
  // none sits behind a branch, and all of them are issued before the first
  // use: the prologue costs about one memory latency.
  const bool b_lds = kRowMajor && (p.r & 7) == 0;  // uniform
  if (b_lds) {
    // direct-to-LDS copy of rows n0 .. n0 + 16 G - 1 of B (1 KB per wave
    // instruction; bytes past B read 0), waited for before the epilogue
    const __amdgpu_buffer_rsrc_t brs0 = bytes_rsrc(p.B + n0 * p.r, 2 * (N - n0) * (int64_t)p.r);
    const int nkb = (int)gemv_b_words(G, p.r) / 256;
    for (int i = wave; i < nkb; i += KW)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          brs0, (__attribute__((address_space(3))) void*)(bsh + 512 * i), 16, 1024 * i + 16 * lane,
          0, 0, 0);
  }
  const int64_t ur = (int64_t)M * p.r;
  const __amdgpu_buffer_rsrc_t urs = bytes_rsrc(p.upart, 4 * kGemvMaxSlices * ur);
  // the slices of U sum e: one 128-byte row (zeros for sums past M r).
  // Kept as raw words until they are added: converting each loaded word to
  // float where it is loaded made the compiler keep only the first word of
  // every 16-byte load.
  auto load_slices = [&](uint32_t (&uv)[kGemvMaxSlices], int64_t e) {
    const int off = e < ur ? (int)(4 * kGemvMaxSlices * e) : kPastEnd;
#pragma unroll
    for (int i = 0; i < kGemvMaxSlices / 4; ++i) {
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(urs, off, 16 * i, 0);
#pragma unroll
      for (int t = 0; t < 4; ++t) uv[4 * i + t] = v[t];
    }
  };
  uint32_t uv[kGemvMaxSlices];
  load_slices(uv, tid);
  if (p.bshift > 0) {
    if constexpr (kLateFirst) issue_first();
    // blocks of 64 << bshift: each 64-element block takes the constant of
    // the block it lies in (rows past N take the last row's)
    const int bs = p.bshift;
    const int64_t cblocks = kblocks >> bs;
    for (int64_t e = tid; e < 16 * G * kblocks; e += NT) {
      const int64_t row = e / kblocks, kb = e - row * kblocks;
      const int64_t n = n0 + row < N ? n0 + row : N - 1;
      const int64_t ci = n * cblocks + (kb >> bs);
      chat_t[row * kbs + kb] = (float)p.q8[ci] * p.step[ci >> 8];
    }
  } else {
    // The workgroup's constants are the contiguous q8 range starting at
    // n0 kblocks, 16 G kblocks bytes long (both multiples of 16), read in
    // 16-byte chunks, kCq per thread per pass.  A chunk starts at a
    // multiple of 16, so its 16 constants share one step (groups of 256).
    // Bytes past the weight's q8 (rows past N, whose results are dropped)
    // read 0.
    // Index math in 32 bits: the workgroup's table has 16 G kblocks < 2^24
    // entries, so an entry index converts to float exactly, and its row
    // (at most 16 G) comes from one multiplication by 1 / kblocks, which
    // is off by well under one; truncating it gives the row or a neighbour,
    // which two comparisons correct.
    constexpr int kCq = 4;
    const int kbl = (int)kblocks;
    const int64_t qtot = N * kblocks;
    const int qbase = (int)(n0 * kblocks);  // < 2^31: q8 is under 2 GiB
    const int nchunk = G * kbl;             // 16 G kblocks / 16
    const int glast = (int)((qtot + 255) >> 8) - 1;
    const __amdgpu_buffer_rsrc_t qrs = bytes_rsrc(p.q8, qtot);
    const int skip = (int)(kbs - kblocks);  // 1 where the row stride is padded
    const float rkb = 1.0f / (float)kbl;
    auto row_of = [&](int e) {  // e / kblocks
      int r = (int)((float)e * rkb);
      const int m = e - r * kbl;
      return m < 0 ? r - 1 : m >= kbl ? r + 1 : r;
    };
    for (int cp = 0; cp < nchunk; cp += kCq * NT) {
      u32x4 qv[kCq];
      float st[kCq];
#pragma unroll
      for (int j = 0; j < kCq; ++j) {
        const int c = cp + tid + j * NT;
        const int o = qbase + 16 * (c < nchunk ? c : nchunk - 1);
        qv[j] = __builtin_amdgcn_raw_buffer_load_b128(qrs, c < nchunk ? o : kPastEnd, 0, 0);
        st[j] = p.step[o >> 8 < glast ? o >> 8 : glast];
      }
      if (kLateFirst && cp == 0) issue_first();
#pragma unroll
      for (int j = 0; j < kCq; ++j) {
        const int c = cp + tid + j * NT;
        if (c < nchunk) {
          // element 16 c + i is block kb0 + i of table row row0, or, from
          // i = kblocks - kb0 on, of the next row (at most one row break
          // per chunk when kblocks >= 16)
          const int row0 = row_of(16 * c), kb0 = 16 * c - row0 * kbl;
          float* const dst = chat_t + row0 * (kbl + skip) + kb0;
          if (kbl >= 16) {  // uniform
            const int brk = kbl - kb0;
#pragma unroll
            for (int i = 0; i < 16; ++i)
              dst[i + (i >= brk ? skip : 0)] =
                  (float)((qv[j][i >> 2] >> (8 * (i & 3))) & 0xffu) * st[j];
          } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int e = 16 * c + i;
              chat_t[e + skip * row_of(e)] =
                  (float)((qv[j][i >> 2] >> (8 * (i & 3))) & 0xffu) * st[j];
            }
          }
        }
      }
    }
  }
  {
    // byte table: thread t writes words t + NT i, i.e. copy t % 16 of
    // entries b = t / 16 + 32 i, whose low code t / 16 % 16 is the same for
    // every i and whose high code t / 256 + 2 i is uniform over the wave
    static_assert(NT == 512 && kLutWords == 8 * NT, "table split assumes 8 waves");
    const float lo = level_of<CT>(p.ut, (tid >> 4) & 15);
    const int hi0 = __builtin_amdgcn_readfirstlane(tid >> 8);
#pragma unroll
    for (int i = 0; i < 8; ++i) lut[tid + NT * i] = pack_bf16x2(lo, level_of<CT>(p.ut, hi0 + 2 * i));
  }
  if (tid < ur) {
    float u = 0.0f;  // slices in order (those past us are zeros)
#pragma unroll
    for (int i = 0; i < kGemvMaxSlices; ++i) u += __builtin_bit_cast(float, uv[i]);
    ush[tid] = u;
  }
  for (int64_t e = tid + NT; e < ur; e += NT) {  // M r > NT: the other sums
    load_slices(uv, e);
    float u = 0.0f;
#pragma unroll
    for (int i = 0; i < kGemvMaxSlices; ++i) u += __builtin_bit_cast(float, uv[i]);
    ush[e] = u;
  }
  __syncthreads();

  if constexpr (kRowMajor) {
    // Row-group-major order: the wave takes its double steps in chunks of
    // DW, and within a chunk one row group after another (all DW double
    // steps of that group's 16 rows), so that the workgroup reads 2 KB of
    // each row of one group at a time instead of 512 bytes of all 16 G rows
    // per step (a read-only stream in this order took 22-26 us at
    // 28672 x 8192 against 27 in the step-major one).  The X fragments of a
    // chunk are loaded once and serve every group; the codes of the next
    // group are in flight while one is consumed (a third slot did not fit
    // in 256 registers with four double steps per chunk).
    // The 2 DW chains (double step j, block h) of group g, software-pipelined
    // as in the step-major order.
    auto compute_g = [&](const Codes& cd, int64_t c, int g) {
      constexpr int NC = 2 * DW;
      const int nvalid = (int)(d1 - DW * c < DW ? d1 - DW * c : DW);  // uniform
      u32x4 cw[DW];
#pragma unroll
      for (int j = 0; j < DW; ++j) {
        u32x4 t;
#pragma unroll
        for (int i = 0; i < 4; ++i) t[i] = nibbles<CT>(cd[j], i);
#pragma unroll
        for (int i = 0; i < 2; ++i) t[i] = __builtin_amdgcn_mov_dpp(t[i], 0xE4, 0xf, 0xf, false);
        const auto s02 = __builtin_amdgcn_permlane32_swap(t[0], t[2], false, false);
        const auto s13 = __builtin_amdgcn_permlane32_swap(t[1], t[3], false, false);
        cw[j] = u32x4{s02[0], s13[0], s02[1], s13[1]};
      }
      u32x4 wl[2][2];
      float ch[2];
      f32x4 pq[2];
      auto lookup = [&](int t) {
        const int j = t >> 1, h = t & 1;
        wl[t & 1][0] = levels8_lut(cw[j][2 * h], lut + i16);
        wl[t & 1][1] = levels8_lut(cw[j][2 * h + 1], lut + i16);
        ch[t & 1] = j < nvalid ? crow_t[g][step_kb(c, j) + h] : 0.0f;
      };
      auto mma = [&](int t) {
        const int j = t >> 1, h = t & 1;
        const f32x4 pb = mfma16(as_bf16x8(xf[j][2 * h]), as_bf16x8(wl[t & 1][0]),
                                f32x4{0.f, 0.f, 0.f, 0.f});
        pq[t & 1] = mfma16(as_bf16x8(xf[j][2 * h + 1]), as_bf16x8(wl[t & 1][1]), pb);
      };
      auto scale = [&](int t) {
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[g][v] += ch[t & 1] * pq[t & 1][v];
      };
      lookup(0);
#pragma unroll
      for (int t = 0; t <= NC; ++t) {
        if (t >= 1) scale(t - 1);
        if (t + 1 < NC) lookup(t + 1);
        if (t < NC) mma(t);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    const int64_t nch = (d1 + DW - 1) / DW;  // 0 for a wave without full steps
    static_assert(G % 2 == 1, "the next chunk's first group goes to slot 1");
    for (int64_t c = 0; c < nch; ++c) {
      issue_x(c);
      // group 0's codes: chunk 0's went out in the prologue, the others
      // during the previous chunk's last group (into slot 1)
      if (c > 0) {
#pragma unroll
        for (int j = 0; j < DW; ++j) cs[0][j] = cs[1][j];
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        // the last group issues the next chunk's first (on the last chunk a
        // clamped re-read of the last step, unused), without a branch so
        // that the wait for this group's codes does not cover those loads
        issue_c(cs[(g + 1) % 2], g + 1 < G ? c : c + 1, g + 1 < G ? g + 1 : 0);
        __builtin_amdgcn_sched_barrier(0);
        compute_g(cs[g % 2], c, g);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  } else {
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
  }
  if (odd_tail) {
    issue(sl[PD - 1], T, true);
    compute(sl[PD - 1], T, true);
  }
  if (b_lds) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the adapter rows are in LDS
  __syncthreads();  // the constant table becomes the reduction buffer

#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int v = 0; v < 4; ++v) red[((wave * G + g) * 4 + v) * 64 + lane] = acc[g][v];
  __syncthreads();

  // Outputs o = tid + NT k: the waves' partial sums added in order, then
  // the LoRA term.  The adapter rows are read JB columns at a time for all
  // of the thread's outputs at once (one latency per JB columns instead of
  // one per output and column batch); columns past r and outputs that are
  // not stored read 0.
  constexpr int KO = (G * 4 * 64 + NT - 1) / NT;
  constexpr int JB = 32;
  const __amdgpu_buffer_rsrc_t brs = bytes_rsrc(p.B, 2 * N * (int64_t)p.r);
  float yk[KO], lk[KO];
  int64_t mk[KO], nk[KO];
  bool vk[KO];
#pragma unroll
  for (int k = 0; k < KO; ++k) {
    const int o = tid + NT * k;
    const int l = o & 63, v = (o >> 6) & 3, g = o >> 8;
    float y = 0.0f;
    if (o < G * 4 * 64) {
#pragma unroll
      for (int w = 0; w < KW; ++w) y += red[((w * G + g) * 4 + v) * 64 + l];
    }
    mk[k] = 4 * (l >> 4) + v;
    nk[k] = n0 + 16 * g + (l & 15);
    vk[k] = o < G * 4 * 64 && mk[k] < M && nk[k] < N;
    yk[k] = y;
    lk[k] = 0.0f;
  }
  if ((p.r & 7) == 0) {
    // r a multiple of 8: 16-byte adapter reads (8 columns, from LDS with
    // seven groups) and 16-byte U reads; JB columns per batch.  Outputs
    // that are not stored read U row 0 and adapter zeros or the first
    // row (their sums are dropped); columns past r are never used.
    for (int j0 = 0; j0 < p.r; j0 += JB) {
      u32x4 bq[KO][JB / 8];
#pragma unroll
      for (int k = 0; k < KO; ++k)
#pragma unroll
        for (int q = 0; q < JB / 8; ++q) {
          const bool jv = j0 + 8 * q < p.r;
          if (b_lds)  // uniform
            bq[k][q] = *reinterpret_cast<const u32x4*>(bsh + (vk[k] ? nk[k] - n0 : 0) * p.r +
                                                       (jv ? j0 + 8 * q : 0));
          else
            bq[k][q] = __builtin_amdgcn_raw_buffer_load_b128(
                brs, vk[k] && jv ? (int)(2 * (nk[k] * p.r + j0 + 8 * q)) : kPastEnd, 0, 0);
        }
      __builtin_amdgcn_sched_barrier(0);  // every load of the batch before the first use
#pragma unroll
      for (int q = 0; q < JB / 8; ++q) {
        if (j0 + 8 * q >= p.r) break;  // uniform
#pragma unroll
        for (int k = 0; k < KO; ++k) {
          const float* ur8 = ush + (vk[k] ? mk[k] * p.r : 0) + j0 + 8 * q;
          const f32x4 u0 = *reinterpret_cast<const f32x4*>(ur8);
          const f32x4 u1 = *reinterpret_cast<const f32x4*>(ur8 + 4);
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const uint32_t wd = bq[k][q][t >> 1];
            const float b = bf16_to_f32((uint16_t)((t & 1) ? wd >> 16 : wd & 0xffffu));
            lk[k] += (t < 4 ? u0[t] : u1[t - 4]) * b;
          }
        }
      }
    }
  } else {
    for (int j0 = 0; j0 < p.r; j0 += JB) {
      uint16_t bv[KO][JB];
#pragma unroll
      for (int k = 0; k < KO; ++k)
#pragma unroll
        for (int t = 0; t < JB; ++t)
          bv[k][t] = __builtin_amdgcn_raw_buffer_load_b16(
              brs, (vk[k] && j0 + t < p.r) ? (int)(2 * (nk[k] * p.r + j0 + t)) : kPastEnd, 0, 0);
#pragma unroll
      for (int k = 0; k < KO; ++k)
        if (vk[k]) {
#pragma unroll
          for (int t = 0; t < JB; ++t)
            if (j0 + t < p.r) lk[k] += ush[mk[k] * p.r + j0 + t] * bf16_to_f32(bv[k][t]);
        }
    }
  }
#pragma unroll
  for (int k = 0; k < KO; ++k)
    if (vk[k]) p.Y[mk[k] * N + nk[k]] = f32_to_bf16(yk[k] + p.s * lk[k]);
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
  static_assert(kGemvMaxSlices == 32, "at most 32 slices below");
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
  (void)K;
  return (size_t)kGemvMaxSlices * M * r * sizeof(float);
}

template <int G>
hipError_t launch_qgemv_g(const GemvArgs& a, int code, hipStream_t stream) {
  // seven row groups run the row-group-major loop; their ring of steps only
  // serves an odd tail block, one slot in flight
  constexpr int KW = 8, PD = G == 7 ? 2 : QN_GEMV_PD;
  const size_t lds = 4 * (size_t)gemv_lds_words(G, KW, a.M, a.r, a.K / 64);
  const dim3 grid((unsigned)((a.N + 16 * G - 1) / (16 * G)));
  return with_any_code(code, [&](auto ct) {
    const void* fn = reinterpret_cast<const void*>(&k_qgemv<G, KW, PD, decltype(ct)>);
    // dynamic LDS above the default 64 KB needs the limit raised; the call is
    // cheap and idempotent, and made for the device the launch goes to
    // (a per-process cache would only cover the first device)
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (G == 7 ? 160 : 96) * 1024);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_qgemv<G, KW, PD, decltype(ct)>), grid, dim3(64 * KW), lds, stream, a);
    return hipGetLastError();
  });
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
  const GemvArgs a{w.codes, w.q8, w.step, X,     M, w.N, w.K,  upart,
                   B,       r,    s,      Y, U_out, w.bshift, w.ut};
  const int64_t kblocks = w.K / 64;
  // 16 G weight rows per workgroup, K split over its 8 waves.
  //  - G = 7 when the 16-row groups make exactly one workgroup of 7 per CU
  //    (a 28672-row weight on 256 CUs): no CU gets more rows than another,
  //    and each CU loads the X fragments once.
  //  - G = 1 for one or two tokens when G = 2 would leave CUs without a
  //    workgroup (fewer than 32 rows per CU): every CU then streams.  With
  //    one workgroup per CU or more, G = 2 is faster (8192 x 8192 on 256
  //    CUs at one token: 15.6 against 17.9 us), and with more tokens the
  //    X fragments, loaded once per workgroup, favour G = 2 further.
  //  - G = 2 otherwise.
  // compute units of the current device, the one the launch goes to
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 0;
  const int64_t groups = (w.N + 15) / 16;
  const bool g7 = cus > 0 && groups % (7 * (int64_t)cus) == 0 &&
                  4 * gemv_lds_words(7, 8, M, r, kblocks) <= 160 * 1024;
  const bool g1 = !g7 && M <= 2 && cus > 0 && groups < 2 * (int64_t)cus;
  e = g7   ? launch_qgemv_g<7>(a, w.code, stream)
      : g1 ? launch_qgemv_g<1>(a, w.code, stream)
           : launch_qgemv_g<2>(a, w.code, stream);
  if (e != hipSuccess) return e;
  if (ev1) e = hipEventRecord(ev1, stream);
  return e;
}

}  // namespace qn
