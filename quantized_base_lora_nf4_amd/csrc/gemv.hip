// Forward pass for few tokens (M <= 16): the whole cost is streaming the
// packed 4-bit weight (codes + 8-bit constants + fp32 steps, 4.13 bits per
// weight) out of HBM once, so the kernel is shaped for bandwidth, not for
// MFMA throughput.
//
// Dequantize-on-the-fly as in "QLoRA: fine-tuning a 65B model on one GPU",
// section "Where the memory goes".  To stay within the VALU budget of a
// memory-bound stream (~2.5 lane-ops per weight at 8 TB/s on 256 CUs), the
// codes are expanded to *unscaled* bf16 levels through a 256-entry byte
// table (one LDS read yields two bf16 values in MFMA operand order), the
// MFMA sums one 64-element block at a time, and the block constant
// fl32(q8 * step) multiplies that block's fp32 partial sum.  The result
// differs from using the bf16-rounded dequantized weight only by the bf16
// rounding of the levels (relative 2^-9 per weight); accumulation is fp32.
//
// Work split: a workgroup of 4 waves owns 64 weight rows and one of S equal
// slices of K; each wave owns 16 rows.  In a 64-column block, lane l reads 8
// bytes (16 codes) of row l % 16 at byte 8 (l / 16); MFMA j (0, 1) of the
// block contracts codes 8 j .. 8 j + 7 of every lane's 16, with the matching
// X elements on the A side.  Every MFMA therefore stays inside one block.
#include "kernels.hpp"

namespace qn {

namespace {

constexpr int kUnroll = 4;  // blocks in flight per lane

__global__ __launch_bounds__(256) void k_qgemv_partial(const uint8_t* __restrict__ codes,
                                                       const uint8_t* __restrict__ q8,
                                                       const float* __restrict__ step,
                                                       const uint16_t* __restrict__ X, int64_t M,
                                                       int64_t N, int64_t K, int64_t blocks_per_split,
                                                       float* __restrict__ part) {
  __shared__ uint32_t lut[256];
  {
    const int b = threadIdx.x;  // byte value -> (level[lo nibble], level[hi nibble]) as bf16
    lut[b] = pack_bf16x2(level_f32(b & 15), level_f32(b >> 4));
  }
  __syncthreads();

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, q = lane >> 4;
  const int64_t kblocks = K >> 6;
  int64_t n = (int64_t)blockIdx.x * 64 + wave * 16 + col;
  const bool nvalid = n < N;
  if (!nvalid) n = N - 1;
  const int64_t kb0 = (int64_t)blockIdx.y * blocks_per_split;
  int64_t kb1 = kb0 + blocks_per_split;
  if (kb1 > kblocks) kb1 = kblocks;

  const bool mvalid = col < M;  // this lane's A-side row
  const uint16_t* xrow = X + (mvalid ? col : 0) * K + q * 16;
  const uint8_t* crow = codes + n * (K >> 1) + q * 8;
  const int64_t blk_row = n * kblocks;

  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  int64_t kb = kb0;
  for (; kb + kUnroll <= kb1; kb += kUnroll) {
    u32x2 cw[kUnroll];
    u32x4 xa[kUnroll][2];
    float chat[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      cw[u] = *reinterpret_cast<const u32x2*>(crow + (kb + u) * 32);
      const int64_t blk = blk_row + kb + u;
      chat[u] = (float)q8[blk] * step[blk >> 8];
#pragma unroll
      for (int j = 0; j < 2; ++j)
        xa[u][j] = mvalid ? *reinterpret_cast<const u32x4*>(xrow + (kb + u) * 64 + j * 8)
                          : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      f32x4 pb = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t w = cw[u][j];
        const u32x4 bw = u32x4{lut[w & 0xffu], lut[(w >> 8) & 0xffu], lut[(w >> 16) & 0xffu],
                               lut[w >> 24]};
        pb = mfma16(as_bf16x8(xa[u][j]), as_bf16x8(bw), pb);
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[v] += chat[u] * pb[v];
    }
  }
  for (; kb < kb1; ++kb) {
    const u32x2 cw = *reinterpret_cast<const u32x2*>(crow + kb * 32);
    const int64_t blk = blk_row + kb;
    const float chat = (float)q8[blk] * step[blk >> 8];
    f32x4 pb = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const u32x4 xa = mvalid ? *reinterpret_cast<const u32x4*>(xrow + kb * 64 + j * 8)
                              : u32x4{0u, 0u, 0u, 0u};
      const uint32_t w = cw[j];
      const u32x4 bw = u32x4{lut[w & 0xffu], lut[(w >> 8) & 0xffu], lut[(w >> 16) & 0xffu],
                             lut[w >> 24]};
      pb = mfma16(as_bf16x8(xa), as_bf16x8(bw), pb);
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[v] += chat * pb[v];
  }

  if (nvalid) {
    float* out = part + (int64_t)blockIdx.y * M * N;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = 4 * q + v;
      if (m < M) out[m * N + n] = acc[v];
    }
  }
}

__global__ __launch_bounds__(256) void k_gemv_finish(const float* __restrict__ part, int splits,
                                                     int64_t M, int64_t N,
                                                     const uint16_t* __restrict__ U, int64_t ldu,
                                                     const uint16_t* __restrict__ B, int32_t r,
                                                     float s, uint16_t* __restrict__ Y) {
  const int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (e >= M * N) return;
  const int64_t m = e / N, n = e - m * N;
  float acc = 0.0f;
  for (int sp = 0; sp < splits; ++sp) acc += part[(int64_t)sp * M * N + e];
  float lora = 0.0f;
  for (int j = 0; j < r; ++j) lora += bf16_to_f32(U[m * ldu + j]) * bf16_to_f32(B[n * r + j]);
  Y[e] = f32_to_bf16(acc + s * lora);
}

}  // namespace

int gemv_splits(int64_t N, int64_t K) {
  const int64_t tiles = (N + 63) / 64;
  const int64_t kblocks = K / 64;
  int64_t s = (768 + tiles - 1) / tiles;  // aim for ~3 workgroups per CU
  const int64_t max_s = (kblocks + 7) / 8;  // keep >= 8 blocks per split
  if (s > max_s) s = max_s;
  if (s < 1) s = 1;
  return (int)s;
}

hipError_t launch_qgemv_partial(const Nf4View& w, const uint16_t* X, int64_t M, int splits,
                                float* part, hipStream_t stream) {
  const int64_t kblocks = w.K / 64;
  const int64_t bps = (kblocks + splits - 1) / splits;
  dim3 grid((unsigned)((w.N + 63) / 64), (unsigned)splits);
  hipLaunchKernelGGL(k_qgemv_partial, grid, dim3(256), 0, stream, w.codes, w.q8, w.step, X, M,
                     w.N, w.K, bps, part);
  return hipGetLastError();
}

hipError_t launch_gemv_finish(const float* part, int splits, int64_t M, int64_t N,
                              const uint16_t* U, int64_t ldu, const uint16_t* B, int32_t r,
                              float s, uint16_t* Y, hipStream_t stream) {
  const int64_t total = M * N;
  hipLaunchKernelGGL(k_gemv_finish, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream,
                     part, splits, M, N, U, ldu, B, r, s, Y);
  return hipGetLastError();
}

}  // namespace qn
