// Fused NF4 + LoRA linear layer: MFMA tile kernels that dequantize the
// frozen weight on chip.
//
// The base weight lives in HBM only as packed 4-bit codes plus 8-bit block
// constants; every forward and backward pass turns the tile it needs into
// bf16 inside LDS and never writes a 16-bit copy back ("QLoRA: fine-tuning
// a 65B model on one GPU", section "Where the memory goes"; the backward
// pass re-materializes the weight from the quantized module as in
// "ModuLoRA: Finetuning 2-Bit LLMs on Consumer GPUs by Integrating with
// Modular Quantizers", abstract).  The LoRA product is folded into the same
// accumulators as extra contraction steps:
//   Y  = [X | s U] [W | B]^T          (forward, contraction over K then r)
//   dX = [dY | dU] [W ; A]            (backward, contraction over N then r)
//
// The dequantized tile is bit-identical to nf4_dequantize:
// w = bf16_rne(level[code] * fl32(q8 * step)).
#include "kernels.hpp"

namespace qn {

namespace {

constexpr int LD = 72;  // LDS row stride in bf16 elements (64 + 8 pad: 144 B)

// One 64-deep slice of MFMA work for a 4-wave workgroup arranged 2 x 2, each
// wave owning a 128 x 64 output tile (4 x 2 tiles of 32 x 32).
// As: [256][LD] rows = output rows, Bs: [128][LD] rows = output columns; both
// store the contraction index contiguously.
__device__ __forceinline__ void mma_slice(const uint16_t* As, const uint16_t* Bs, int wm, int wn,
                                          int lane, f32x16 (&acc)[4][2]) {
  const int r32 = lane & 31;
  const int kh = (lane >> 5) * 8;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    bf16x8 a[4], b[2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      a[i] = *reinterpret_cast<const bf16x8*>(As + (wm * 128 + i * 32 + r32) * LD + kk * 16 + kh);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      b[j] = *reinterpret_cast<const bf16x8*>(Bs + (wn * 64 + j * 32 + r32) * LD + kk * 16 + kh);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(a[i], b[j], acc[i][j]);
  }
}

// Store a 256 x 128 fp32 accumulator tile as bf16 into out[row][col] with row
// stride ld, skipping rows >= rows and columns >= cols.
__device__ __forceinline__ void store_tile(uint16_t* out, int64_t ld, int64_t row0, int64_t col0,
                                           int64_t rows, int64_t cols, int wm, int wn, int lane,
                                           const f32x16 (&acc)[4][2]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = col0 + wn * 64 + j * 32 + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = row0 + wm * 128 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (row < rows && col < cols) out[row * ld + col] = f32_to_bf16(acc[i][j][v]);
      }
    }
}

// Eight NF4 codes (one 32-bit word, element order = nibble order) scaled by
// chat, as four packed bf16 pairs.
__device__ __forceinline__ u32x4 dequant8(uint32_t w, float chat, const float* lv) {
  u32x4 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float lo = lv[(w >> (8 * j)) & 15u] * chat;
    const float hi = lv[(w >> (8 * j + 4)) & 15u] * chat;
    o[j] = pack_bf16x2(lo, hi);
  }
  return o;
}

// Stage a 256 x 64 tile of a bf16 matrix with zero-padded columns (row
// stride ld, a multiple of 8; the tile's columns c0..c0+63 all exist) into
// As, multiplying by `scale` in fp32 and rounding back to bf16 when scale != 1.
__device__ __forceinline__ void stage_rows_scaled(uint16_t* As, const uint16_t* src, int64_t ld,
                                                  int64_t row0, int64_t rows, int64_t c0,
                                                  float scale, bool do_scale, int tid) {
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int e = tid + 256 * q;
    const int row = e >> 3, c8 = e & 7;
    int64_t gr = row0 + row;
    if (gr >= rows) gr = rows - 1;
    u32x4 v = *reinterpret_cast<const u32x4*>(src + gr * ld + c0 + c8 * 8);
    if (do_scale) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        v[j] = pack_bf16x2(bf16_lo_to_f32(v[j]) * scale, bf16_hi_to_f32(v[j]) * scale);
    }
    *reinterpret_cast<u32x4*>(As + row * LD + c8 * 8) = v;
  }
}

// ---------------------------------------------------------------------------
// Forward
// ---------------------------------------------------------------------------
struct FwdArgs {
  const uint16_t* X;
  const uint8_t* codes;
  const uint8_t* q8;
  const float* step;
  const uint16_t* U;
  int64_t ldu;
  const uint16_t* B;
  int32_t r;
  float s;
  uint16_t* Y;
  int64_t M, N, K;
};

__global__ __launch_bounds__(256, 2) void k_qgemm_fwd(FwdArgs p) {
  __shared__ __attribute__((aligned(16))) uint16_t As[256 * LD];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[128 * LD];
  __shared__ float lv[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = (int64_t)blockIdx.y * 256, n0 = (int64_t)blockIdx.x * 128;
  const int64_t M = p.M, N = p.N, K = p.K;
  const int64_t kblocks = K >> 6;
  if (tid < 16) lv[tid] = level_f32(tid);

  // X loader: 8 chunks of 16 B per thread, 8 consecutive threads per row.
  // W loader: thread -> (row tid/2, half tid%2): 32 codes = 16 bytes.
  const int wrow = tid >> 1, whalf = tid & 1;
  int64_t gn = n0 + wrow;
  if (gn >= N) gn = N - 1;
  const uint8_t* wcodes = p.codes + gn * (K >> 1) + whalf * 16;
  const int64_t wblk0 = gn * kblocks;

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  u32x4 xr[8];
  u32x4 wr;
  float chat_r;
  auto load = [&](int64_t kt) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int e = tid + 256 * q;
      int64_t gm = m0 + (e >> 3);
      if (gm >= M) gm = M - 1;
      xr[q] = *reinterpret_cast<const u32x4*>(p.X + gm * K + kt * 64 + (e & 7) * 8);
    }
    wr = *reinterpret_cast<const u32x4*>(wcodes + kt * 32);
    const int64_t blk = wblk0 + kt;
    chat_r = (float)p.q8[blk] * p.step[blk >> 8];
  };
  auto stage = [&]() {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int e = tid + 256 * q;
      *reinterpret_cast<u32x4*>(As + (e >> 3) * LD + (e & 7) * 8) = xr[q];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<u32x4*>(Bs + wrow * LD + whalf * 32 + j * 8) = dequant8(wr[j], chat_r, lv);
  };

  load(0);
  __syncthreads();  // lv ready
  for (int64_t kt = 0; kt < kblocks; ++kt) {
    stage();
    __syncthreads();
    if (kt + 1 < kblocks) load(kt + 1);
    mma_slice(As, Bs, wm, wn, lane, acc);
    __syncthreads();
  }

  // LoRA: extra contraction over r with A-side bf16(s U) and B-side B.
  const bool bvec = (p.r & 7) == 0;
  for (int j0 = 0; j0 < p.r; j0 += 64) {
    stage_rows_scaled(As, p.U, p.ldu, m0, M, j0, p.s, true, tid);
    if (bvec) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = tid + 256 * q;
        const int row = e >> 3, c8 = e & 7;
        int64_t g = n0 + row;
        if (g >= N) g = N - 1;
        u32x4 v = u32x4{0u, 0u, 0u, 0u};
        if (j0 + c8 * 8 < p.r) v = *reinterpret_cast<const u32x4*>(p.B + g * p.r + j0 + c8 * 8);
        *reinterpret_cast<u32x4*>(Bs + row * LD + c8 * 8) = v;
      }
    } else {
      for (int e = tid; e < 128 * 64; e += 256) {
        const int row = e >> 6, c = e & 63;
        int64_t g = n0 + row;
        if (g >= N) g = N - 1;
        const int jj = j0 + c;
        Bs[row * LD + c] = (jj < p.r) ? p.B[g * p.r + jj] : (uint16_t)0;
      }
    }
    __syncthreads();
    mma_slice(As, Bs, wm, wn, lane, acc);
    __syncthreads();
  }

  store_tile(p.Y, N, m0, n0, M, N, wm, wn, lane, acc);
}

// ---------------------------------------------------------------------------
// Backward (dX)
// ---------------------------------------------------------------------------
struct BwdArgs {
  const uint16_t* dY;
  const uint8_t* codes;
  const uint8_t* q8;
  const float* step;
  const uint16_t* dU;
  int64_t lddu;
  const uint16_t* A;
  int32_t r;
  uint16_t* dX;
  int64_t M, N, K;
};

// Output tile 256 (tokens) x 128 (input features); contraction over the
// weight's rows in slices of 64.  The weight slice (64 rows x 128 columns)
// is dequantized transposed into Bs[column][row] so that the MFMA B operand
// reads 8 consecutive rows.
__global__ __launch_bounds__(256, 2) void k_qgemm_bwd(BwdArgs p) {
  __shared__ __attribute__((aligned(16))) uint16_t As[256 * LD];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[128 * LD];
  __shared__ float lv[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = (int64_t)blockIdx.y * 256, k0 = (int64_t)blockIdx.x * 128;
  const int64_t M = p.M, N = p.N, K = p.K;
  const int64_t kblocks = K >> 6;
  const int64_t nsteps = (N + 63) >> 6;
  if (tid < 16) lv[tid] = level_f32(tid);

  // W loader: thread -> rows 4*rg .. 4*rg+3 of the slice, columns 8*cg .. 8*cg+7.
  const int rg = tid >> 4, cg = tid & 15;
  const int64_t kcol = k0 + cg * 8;
  const bool kvalid = kcol < K;

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  u32x4 dr[8];
  uint32_t wr[4];
  float chat_r[4];
  auto load = [&](int64_t ns) {
    const int64_t nc = ns * 64;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int e = tid + 256 * q;
      int64_t gm = m0 + (e >> 3);
      if (gm >= M) gm = M - 1;
      const int64_t col = nc + (e & 7) * 8;
      dr[q] = (col < N) ? *reinterpret_cast<const u32x4*>(p.dY + gm * N + col)
                        : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int64_t n = nc + rg * 4 + rr;
      if (n < N && kvalid) {
        wr[rr] = *reinterpret_cast<const uint32_t*>(p.codes + ((n * K + kcol) >> 1));
        const int64_t blk = n * kblocks + (kcol >> 6);
        chat_r[rr] = (float)p.q8[blk] * p.step[blk >> 8];
      } else {
        wr[rr] = 0u;
        chat_r[rr] = 0.0f;
      }
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int e = tid + 256 * q;
      *reinterpret_cast<u32x4*>(As + (e >> 3) * LD + (e & 7) * 8) = dr[q];
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float v[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) v[rr] = lv[(wr[rr] >> (4 * c)) & 15u] * chat_r[rr];
      u32x2 o = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      *reinterpret_cast<u32x2*>(Bs + (cg * 8 + c) * LD + rg * 4) = o;
    }
  };

  load(0);
  __syncthreads();
  for (int64_t ns = 0; ns < nsteps; ++ns) {
    stage();
    __syncthreads();
    if (ns + 1 < nsteps) load(ns + 1);
    mma_slice(As, Bs, wm, wn, lane, acc);
    __syncthreads();
  }

  // LoRA: dX += dU A, contraction over r.  A[j][k] is staged transposed.
  for (int j0 = 0; j0 < p.r; j0 += 64) {
    stage_rows_scaled(As, p.dU, p.lddu, m0, M, j0, 1.0f, false, tid);
    for (int e = tid; e < 64 * 16; e += 256) {
      const int jr = e >> 4, c8 = e & 15;  // adapter row j0+jr, columns 8*c8..
      const int64_t col = k0 + c8 * 8;
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (j0 + jr < p.r && col < K) v = *reinterpret_cast<const u32x4*>(p.A + (j0 + jr) * K + col);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        Bs[(c8 * 8 + 2 * q) * LD + jr] = (uint16_t)(v[q] & 0xffffu);
        Bs[(c8 * 8 + 2 * q + 1) * LD + jr] = (uint16_t)(v[q] >> 16);
      }
    }
    __syncthreads();
    mma_slice(As, Bs, wm, wn, lane, acc);
    __syncthreads();
  }

  store_tile(p.dX, K, m0, k0, M, K, wm, wn, lane, acc);
}

}  // namespace

hipError_t launch_qgemm_fwd(const Nf4View& w, const uint16_t* X, int64_t M, const uint16_t* U,
                            int64_t ldu, const uint16_t* B, int32_t r, float s, uint16_t* Y,
                            hipStream_t stream) {
  FwdArgs a{X, w.codes, w.q8, w.step, U, ldu, B, r, s, Y, M, w.N, w.K};
  dim3 grid((unsigned)((w.N + 127) / 128), (unsigned)((M + 255) / 256));
  hipLaunchKernelGGL(k_qgemm_fwd, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_qgemm_bwd(const Nf4View& w, const uint16_t* dY, int64_t M, const uint16_t* dU,
                            int64_t lddu, const uint16_t* A, int32_t r, uint16_t* dX,
                            hipStream_t stream) {
  BwdArgs a{dY, w.codes, w.q8, w.step, dU, lddu, A, r, dX, M, w.N, w.K};
  dim3 grid((unsigned)((w.K + 127) / 128), (unsigned)((M + 255) / 256));
  hipLaunchKernelGGL(k_qgemm_bwd, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace qn
