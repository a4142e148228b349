// Small-rank LoRA products: U = X A^T, dU = s dY B, dB = s dY^T U and
// dA = dU^T X.  LoRA trains only a low-rank pair beside the frozen weight
// ("QLoRA: fine-tuning a 65B model on one GPU", section "Where the memory
// goes"), so one side of each of these products is the rank r (<= 256) and
// the contraction is long (K, N or M).
//
// One generic MFMA kernel computes C[I, J] = sum_c Aop(i, c) Bop(c, j) over
// a slice of the contraction and writes fp32 partial sums; a second kernel
// adds the slices in a fixed order, scales and rounds to bf16.  No atomics,
// so results are bit-reproducible.
//
// Tiles are 64 x 64 outputs per 256-thread workgroup (2 x 2 waves of one
// 32 x 32 MFMA tile each), 64-deep contraction steps staged through LDS.
// Operands are read element-wise with the thread order chosen so that
// consecutive lanes touch consecutive addresses in whichever dimension is
// contiguous.
#include "kernels.hpp"

namespace qn {

namespace {

constexpr int SLD = 72;
constexpr int kSkinnyStep = 64;

struct SkinnyArgs {
  SkinnyOp op;
  int64_t c_split;  // contraction length per split (multiple of 64)
  float* part;
  bool a_vec, b_vec;
};

// Stage a 64 x 64 operand tile into T[x][c] (c contiguous in LDS).
// Element (x, c) is at src[x * sx + c * sc]; rows x >= X or columns
// c >= cend are zero.  One of sx, sc is 1.  When the other stride and the
// base are 16-byte aligned (`vec`), every thread moves two 16-byte chunks of
// eight contiguous elements: along c they go to LDS as one 16-byte store;
// along x they are scattered as eight 2-byte stores (the transpose).
// Otherwise elements are moved one at a time.  The contraction length of
// every caller is a multiple of 8, so a chunk is either wholly inside or
// wholly outside [c0, cend) and [0, X) when X is a multiple of 8.
__device__ __forceinline__ void stage_op(uint16_t* T, const uint16_t* src, int64_t sx, int64_t sc,
                                         int64_t x0, int64_t X, int64_t c0, int64_t cend,
                                         bool vec, int tid) {
  const bool c_fast = (sc == 1);
  if (vec) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int e = tid + 256 * q;
      if (c_fast) {
        const int xi = e >> 3, ci = (e & 7) * 8;
        const int64_t gx = x0 + xi, gc = c0 + ci;
        u32x4 v = u32x4{0u, 0u, 0u, 0u};
        if (gx < X && gc < cend) v = *reinterpret_cast<const u32x4*>(src + gx * sx + gc);
        *reinterpret_cast<u32x4*>(T + xi * SLD + ci) = v;
      } else {
        const int ci = e >> 3, xi = (e & 7) * 8;
        const int64_t gx = x0 + xi, gc = c0 + ci;
        u32x4 v = u32x4{0u, 0u, 0u, 0u};
        if (gx < X && gc < cend) v = *reinterpret_cast<const u32x4*>(src + gc * sc + gx);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          T[(xi + 2 * j) * SLD + ci] = (uint16_t)(v[j] & 0xffffu);
          T[(xi + 2 * j + 1) * SLD + ci] = (uint16_t)(v[j] >> 16);
        }
      }
    }
    return;
  }
#pragma unroll 4
  for (int q = 0; q < 16; ++q) {
    const int e = tid + 256 * q;
    const int xi = c_fast ? (e >> 6) : (e & 63);
    const int ci = c_fast ? (e & 63) : (e >> 6);
    const int64_t gx = x0 + xi, gc = c0 + ci;
    uint16_t v = 0;
    if (gx < X && gc < cend) v = src[gx * sx + gc * sc];
    T[xi * SLD + ci] = v;
  }
}

__global__ __launch_bounds__(256) void k_skinny_partial(SkinnyArgs p) {
  __shared__ __attribute__((aligned(16))) uint16_t As[64 * SLD];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[64 * SLD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wi = wave >> 1, wj = wave & 1;
  const int64_t j0 = (int64_t)blockIdx.x * 64, i0 = (int64_t)blockIdx.y * 64;
  const int64_t cs = (int64_t)blockIdx.z * p.c_split;
  int64_t ce = cs + p.c_split;
  if (ce > p.op.C) ce = p.op.C;
  const SkinnyOp& op = p.op;

  f32x16 acc = f32x16{};
  const int r32 = lane & 31, kh = (lane >> 5) * 8;
  for (int64_t c0 = cs; c0 < ce; c0 += kSkinnyStep) {
    stage_op(As, op.a, op.a_si, op.a_sc, i0, op.I, c0, ce, p.a_vec, tid);
    stage_op(Bs, op.b, op.b_sj, op.b_sc, j0, op.J, c0, ce, p.b_vec, tid);
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(As + (wi * 32 + r32) * SLD + kk * 16 + kh);
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(Bs + (wj * 32 + r32) * SLD + kk * 16 + kh);
      acc = mfma32(a, b, acc);
    }
    __syncthreads();
  }

  float* out = p.part + (int64_t)blockIdx.z * op.I * op.J;
  const int64_t j = j0 + wj * 32 + r32;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int64_t i = i0 + wi * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
    if (i < op.I && j < op.J) out[i * op.J + j] = acc[v];
  }
}

__global__ __launch_bounds__(256) void k_skinny_finish(const float* __restrict__ part, int splits,
                                                       int64_t I, int64_t J, float scale,
                                                       uint16_t* __restrict__ out, int64_t o_si,
                                                       int64_t Jw, uint16_t* __restrict__ out2,
                                                       int64_t o2_si) {
  const int64_t total = I * Jw;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = e / Jw, j = e - i * Jw;
    if (j < J) {
      float acc = 0.0f;
      for (int s = 0; s < splits; ++s) acc += part[(int64_t)s * I * J + i * J + j];
      const uint16_t v = f32_to_bf16(acc * scale);
      out[i * o_si + j] = v;
      if (out2) out2[i * o2_si + j] = v;
    } else {
      out[i * o_si + j] = 0;
    }
  }
}

}  // namespace

int skinny_splits(int64_t I, int64_t J, int64_t C) {
  const int64_t tiles = ((I + 63) / 64) * ((J + 63) / 64);
  const int64_t steps = (C + kSkinnyStep - 1) / kSkinnyStep;
  int64_t s = (1024 + tiles - 1) / tiles;  // aim for ~4 workgroups per CU
  const int64_t max_s = (steps + 3) / 4;   // at least 4 steps per split
  if (s > max_s) s = max_s;
  if (s < 1) s = 1;
  if (s > 64) s = 64;
  return (int)s;
}

static int64_t split_len(int64_t C, int s) {
  const int64_t steps = (C + kSkinnyStep - 1) / kSkinnyStep;
  return ((steps + s - 1) / s) * kSkinnyStep;
}

size_t skinny_partial_bytes(int64_t I, int64_t J, int64_t C) {
  const int s = skinny_splits(I, J, C);
  return (size_t)s * (size_t)I * (size_t)J * sizeof(float);
}

hipError_t launch_skinny_partial(const SkinnyOp& op, int splits, float* part, hipStream_t stream) {
  const int64_t cl = split_len(op.C, splits);
  // 16-byte chunks need an aligned base and an aligned outer stride, a
  // contraction length that is a multiple of 8 and (for chunks along the
  // output dimension) an output extent that is a multiple of 8.
  auto vec_ok = [&](const uint16_t* ptr, int64_t sx, int64_t sc, int64_t X) {
    const int64_t outer = (sc == 1) ? sx : sc;
    const bool along_x = (sc != 1);
    return ((uintptr_t)ptr & 15u) == 0 && (outer % 8) == 0 && (op.C % 8) == 0 &&
           (!along_x || (X % 8) == 0);
  };
  SkinnyArgs a{op, cl, part, vec_ok(op.a, op.a_si, op.a_sc, op.I), vec_ok(op.b, op.b_sj, op.b_sc, op.J)};
  dim3 grid((unsigned)((op.J + 63) / 64), (unsigned)((op.I + 63) / 64), (unsigned)splits);
  hipLaunchKernelGGL(k_skinny_partial, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_skinny_finish(const float* part, int splits, int64_t I, int64_t J, float scale,
                                uint16_t* out, int64_t o_si, int64_t Jw, uint16_t* out2,
                                int64_t o2_si, hipStream_t stream) {
  const int64_t total = I * Jw;
  int64_t grid = (total + 255) / 256;
  if (grid > 16384) grid = 16384;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(k_skinny_finish, dim3((unsigned)grid), dim3(256), 0, stream, part, splits, I,
                     J, scale, out, o_si, Jw, out2, o2_si);
  return hipGetLastError();
}

}  // namespace qn
