// Per-matrix quantization configuration under a memory budget ("LQ-LoRA:
// Low-rank Plus Quantized Matrix Decomposition for Efficient Language Model
// Finetuning", abstract: an integer linear program chooses each matrix's
// quantization parameters for an overall memory budget).
//
// Device side: the error of one configuration on one matrix,
// ||R - W_hat(R)||_F^2 with R = W or W - L1 L2t^T, from the block quantizer
// and a fused dequantize-and-square pass with a fixed-order fp64 sum.
// Host side: the program itself (choose one configuration per matrix,
// minimize the total error, total bytes within the budget), solved exactly
// as a multiple-choice knapsack by dynamic programming over Pareto fronts.
#include <algorithm>
#include <vector>

#include "kernels.hpp"

namespace qn {
namespace {

constexpr int kErrBlocks = 1024;  // fixed grid: the partial count never changes

// Per-workgroup partial sums of (R - W_hat)^2 in fp64: each thread walks
// groups of eight weights (grid-stride), then a fixed tree in LDS.
template <class CT>
__global__ __launch_bounds__(256) void k_sq_error(const float* __restrict__ R,
                                                  const uint8_t* __restrict__ codes,
                                                  const uint8_t* __restrict__ q8,
                                                  const float* __restrict__ step, int64_t n8,
                                                  int bshift, double* __restrict__ part) {
  __shared__ float lv[16];
  __shared__ double red[256];
  if (threadIdx.x < 16) lv[threadIdx.x] = code_value<CT>(threadIdx.x);
  __syncthreads();
  double acc = 0.0;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n8;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t b = i >> 3;
    uint32_t w;
    if constexpr (CT::kBits == 4) {
      w = *reinterpret_cast<const uint32_t*>(codes + i * 4);
    } else {
      w = nibbles<CT>(load_half<CT>(codes + b * block_bytes<CT>() + ((i >> 2) & 1) * half_bytes<CT>()),
                      (int)(i & 3));
    }
    const int64_t cb = b >> bshift;  // the block of 64 << bshift elements
    const float chat = (float)q8[cb] * step[cb >> 8];
    const f32x4 r0 = *reinterpret_cast<const f32x4*>(R + i * 8);
    const f32x4 r1 = *reinterpret_cast<const f32x4*>(R + i * 8 + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const double d0 = (double)r0[j] - (double)bf16_to_f32(f32_to_bf16(lv[(w >> (4 * j)) & 15u] * chat));
      const double d1 =
          (double)r1[j] - (double)bf16_to_f32(f32_to_bf16(lv[(w >> (4 * j + 16)) & 15u] * chat));
      acc = fma(d0, d0, acc);
      acc = fma(d1, d1, acc);
    }
  }
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int w2 = 128; w2 > 0; w2 >>= 1) {
    if ((int)threadIdx.x < w2) red[threadIdx.x] += red[threadIdx.x + w2];
    __syncthreads();
  }
  if (threadIdx.x == 0) part[blockIdx.x] = red[0];
}

// out = sum of the kErrBlocks partials: thread t adds partials 4 t .. 4 t + 3
// in order, then a fixed tree in LDS (the same order on every call).
__global__ __launch_bounds__(256) void k_sq_error_sum(const double* __restrict__ part,
                                                      double* __restrict__ out) {
  static_assert(kErrBlocks == 4 * 256, "four partials per thread");
  __shared__ double red[256];
  const int t = threadIdx.x;
  red[t] = ((part[4 * t] + part[4 * t + 1]) + part[4 * t + 2]) + part[4 * t + 3];
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (t < w) red[t] += red[t + w];
    __syncthreads();
  }
  if (t == 0) *out = red[0];
}

inline size_t al(size_t v) { return (v + 255) / 256 * 256; }

struct ErrPlan {
  size_t r_off, codes_off, q8_off, step_off, part_off, total;
};

ErrPlan err_plan(int64_t N, int64_t K, int bits, int bshift, bool lowrank) {
  ErrPlan p{};
  size_t o = 0;
  auto take = [&](size_t b) {
    const size_t at = o;
    o += al(b);
    return at;
  };
  const int64_t nb = N * K / (64 << bshift);
  p.r_off = lowrank ? take(4 * (size_t)N * K) : 0;
  p.codes_off = take((size_t)(N * K / 8 * bits));
  p.q8_off = take((size_t)nb);
  p.step_off = take(4 * (size_t)((nb + 255) / 256));
  p.part_off = take(8 * (size_t)kErrBlocks);
  p.total = o;
  return p;
}

}  // namespace

size_t quant_error_workspace_bytes(int64_t N, int64_t K, int bits, int bshift, bool lowrank) {
  return err_plan(N, K, bits, bshift, lowrank).total;
}

hipError_t launch_quant_error(const float* W, int64_t N, int64_t K, int code, int bshift,
                              const float* L1, const float* L2t, int r, double* sq_err, void* ws,
                              hipStream_t stream) {
  const int bits = with_code(code, [](auto ct) { return decltype(ct)::kBits; });
  const bool lowrank = L1 != nullptr;
  const ErrPlan pl = err_plan(N, K, bits, bshift, lowrank);
  char* base = static_cast<char*>(ws);
  const float* R = W;
  if (lowrank) {
    float* Rb = reinterpret_cast<float*>(base + pl.r_off);
    const hipError_t e = launch_lq_residual(W, L1, L2t, N, K, r, Rb, stream);
    if (e != hipSuccess) return e;
    R = Rb;
  }
  uint8_t* codes = reinterpret_cast<uint8_t*>(base + pl.codes_off);
  uint8_t* q8 = reinterpret_cast<uint8_t*>(base + pl.q8_off);
  float* step = reinterpret_cast<float*>(base + pl.step_off);
  double* part = reinterpret_cast<double*>(base + pl.part_off);
  hipError_t e =
      launch_nf4_quantize(R, N * K / (64 << bshift), codes, q8, step, code, bshift, nullptr,
                          stream);
  if (e != hipSuccess) return e;
  with_code(code, [&](auto ct) {
    hipLaunchKernelGGL(k_sq_error<decltype(ct)>, dim3(kErrBlocks), dim3(256), 0, stream, R, codes,
                       q8, step, N * K / 8, bshift, part);
    return 0;
  });
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_sq_error_sum, dim3(1), dim3(256), 0, stream, part, sq_err);
  return hipGetLastError();
}

// Exact solution of: choose c_m for each matrix m, minimize sum_m err[m][c_m]
// subject to sum_m bytes[m][c_m] <= budget.  Matrices are taken in order;
// the partial choices form a front sorted by bytes, and a partial choice is
// dropped when another one has at most its bytes and at most its error
// (every completion of the first is then at least as good: the same suffix
// adds the same bytes and, in the same summation order, no more error), or
// when even the smallest configurations of the remaining matrices no longer
// fit.  Ties are resolved as (error, bytes, choice vector lexicographically).
// Returns false if nothing fits.
bool ilp_plan(int M, int C, const double* err, const int64_t* bytes, int64_t budget,
              int32_t* choice, double* total_err, int64_t* total_bytes) {
  struct Pt {
    int64_t b;
    double e;
    std::vector<int32_t> ch;
  };
  std::vector<int64_t> tail_min(M + 1, 0);  // smallest bytes of matrices m..M-1
  for (int m = M - 1; m >= 0; --m) {
    int64_t mn = bytes[(size_t)m * C];
    for (int c = 1; c < C; ++c) mn = std::min(mn, bytes[(size_t)m * C + c]);
    tail_min[m] = tail_min[m + 1] + mn;
  }
  std::vector<Pt> front{Pt{0, 0.0, {}}};
  for (int m = 0; m < M; ++m) {
    std::vector<Pt> nx;
    nx.reserve(front.size() * C);
    for (const Pt& p : front)
      for (int c = 0; c < C; ++c) {
        const int64_t b = p.b + bytes[(size_t)m * C + c];
        if (b + tail_min[m + 1] > budget) continue;
        Pt q{b, p.e + err[(size_t)m * C + c], p.ch};
        q.ch.push_back(c);
        nx.push_back(std::move(q));
      }
    std::sort(nx.begin(), nx.end(), [](const Pt& a, const Pt& b) {
      if (a.b != b.b) return a.b < b.b;
      if (a.e != b.e) return a.e < b.e;
      return a.ch < b.ch;
    });
    front.clear();
    for (Pt& p : nx)
      if (front.empty() || p.e < front.back().e) front.push_back(std::move(p));
    if (front.empty()) return false;
  }
  const Pt& best = front.back();  // errors fall strictly along the front
  for (int m = 0; m < M; ++m) choice[m] = best.ch[m];
  *total_err = best.e;
  *total_bytes = best.b;
  return true;
}

}  // namespace qn
