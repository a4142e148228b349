// Low-rank plus quantized decomposition of a frozen weight, W ~ Q + L1 L2
// ("LQ-LoRA: Low-rank Plus Quantized Matrix Decomposition for Efficient
// Language Model Finetuning", abstract: the weight becomes, by an iteration,
// a frozen quantized part plus a high-precision low-rank part that finetuning
// trains as the adapter).
//
// Alternating minimization of ||W - Q - L1 L2||_F:
//   L step  rank-r approximation of E = W - Q: randomized subspace iteration
//           from the caller's Gaussian test matrix Omega [K, l] (Halko,
//           Martinsson and Tropp 2011, algorithm 4.4), then Rayleigh-Ritz on
//           the l-dimensional subspace;
//   Q step  the block quantizer (nf4_quant.hip) on R = W - L1 L2.
//
// Kernels (all fp32 data, fp64 for the l x l Gram matrices, their Cholesky
// factors and eigenvectors).  Orthonormal bases come from the Cholesky
// factor of the Gram matrix (the oracle takes its eigenvectors instead:
// both are bases of the same span, and L1 L2 depends on the spans only).
//   k_lq_residual   R = W - L1 L2t^T                    (tiles, HBM + VALU)
//   k_lq_error      E = W - W_hat(Q)                    (elementwise, HBM)
//   k_lq_mul        partial Y = E X or Z = E^T Y over contraction slices
//                   (E streamed once per product)
//   k_lq_reduce     sum of the slices, fixed order
//   k_lq_gram       partial X^T X over row slices, fp64
//   k_lq_chol       Cholesky factor of a Gram matrix G = L L^T
//   k_lq_trsm       X L^{-T} (orthonormal columns), one thread per row
//   k_lq_eig        Jacobi eigenvectors of an l x l matrix (Ritz step)
//   k_lq_mul_xm     Y = X M      [T,l] x [l,c]
//   k_lq_adapter    A = bf16(L2), B = bf16(L1 / s)
// No atomics: every sum has a fixed order, so results are reproducible.
#include <type_traits>

#include "kernels.hpp"

namespace qn {
namespace {

constexpr int kLqMaxL = 96;
constexpr double kDrop = 1e-10;  // relative eigenvalue below which a direction is dropped

// ---------------------------------------------------------------------------
// R = W - L1 L2t^T.  64 x 64 output tile per workgroup, 4 x 4 per thread;
// the tile's L1 rows and L2t rows (r <= 95 values each) staged in LDS.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_lq_residual(const float* __restrict__ W,
                                                     const float* __restrict__ L1,
                                                     const float* __restrict__ L2t, int64_t N,
                                                     int64_t K, int r, float* __restrict__ R) {
  __shared__ float s1[64 * (kLqMaxL + 1)];
  __shared__ float s2[64 * (kLqMaxL + 1)];
  const int st = r | 1;  // odd row stride
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int64_t tiles_k = K / 64;
  const int64_t n0 = (int64_t)(blockIdx.x / tiles_k) * 64, k0 = (int64_t)(blockIdx.x % tiles_k) * 64;
  for (int e = tid; e < 64 * r; e += 256) {
    const int row = e / r, j = e - row * r;
    int64_t n = n0 + row;
    if (n >= N) n = N - 1;
    s1[row * st + j] = L1[n * r + j];
    s2[row * st + j] = L2t[(k0 + row) * r + j];
  }
  __syncthreads();
  float acc[4][4] = {};
  for (int j = 0; j < r; ++j) {
    float a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = s1[(ty * 4 + i) * st + j];
#pragma unroll
    for (int c = 0; c < 4; ++c) b[c] = s2[(tx * 4 + c) * st + j];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[i][c] = fmaf(a[i], b[c], acc[i][c]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t n = n0 + ty * 4 + i;
    if (n >= N) continue;
    const f32x4 w = *reinterpret_cast<const f32x4*>(W + n * K + k0 + tx * 4);
    f32x4 o;
#pragma unroll
    for (int c = 0; c < 4; ++c) o[c] = w[c] - acc[i][c];
    *reinterpret_cast<f32x4*>(R + n * K + k0 + tx * 4) = o;
  }
}

// ---------------------------------------------------------------------------
// E = W - W_hat: eight weights per thread, W_hat as in the dequantizer.
// ---------------------------------------------------------------------------
template <class CT>
__global__ __launch_bounds__(256) void k_lq_error(const float* __restrict__ W,
                                                  const uint8_t* __restrict__ codes,
                                                  const uint8_t* __restrict__ q8,
                                                  const float* __restrict__ step, int64_t n8,
                                                  float* __restrict__ E) {
  __shared__ float lv[16];
  if (threadIdx.x < 16) lv[threadIdx.x] = code_value<CT>(threadIdx.x);
  __syncthreads();
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
    const float chat = (float)q8[b] * step[b >> 8];
    const f32x4 w0 = *reinterpret_cast<const f32x4*>(W + i * 8);
    const f32x4 w1 = *reinterpret_cast<const f32x4*>(W + i * 8 + 4);
    f32x4 o0, o1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float v0 = bf16_to_f32(f32_to_bf16(lv[(w >> (4 * j)) & 15u] * chat));
      const float v1 = bf16_to_f32(f32_to_bf16(lv[(w >> (4 * j + 16)) & 15u] * chat));
      o0[j] = w0[j] - v0;
      o1[j] = w1[j] - v1;
    }
    *reinterpret_cast<f32x4*>(E + i * 8) = o0;
    *reinterpret_cast<f32x4*>(E + i * 8 + 4) = o1;
  }
}

// ---------------------------------------------------------------------------
// The two products with E: Y = E X ([N,K] x [K,l]) and Z = E^T Y
// ([K,N] x [N,l]).  Both stream E once and share one inner loop: a
// workgroup owns 64 rows of the output (rows of E for E X, columns of E for
// E^T Y) and all l columns, for one slice of the contraction; thread
// (rg, cg) accumulates output rows 4 rg .. 4 rg + 3 and columns
// cg CP .. cg CP + CP - 1 (CP = l / 16).  Per 32-deep chunk the operands sit
// in LDS as sa[kk][64] (the four rows of a thread are one 16-byte read) and
// sb[kk][l]; the next chunk's global loads are issued before the current
// chunk's products.  Slices write fp32 partials that k_lq_reduce sums in
// slice order.
// ---------------------------------------------------------------------------
constexpr int kSA = 68;  // row stride of sa (floats)

template <int CP>
__device__ __forceinline__ void chunk_products(const float* sa, const float* sb, int l, int rg,
                                               int cg, float (&acc)[4][6]) {
#pragma unroll 8
  for (int kk = 0; kk < 32; ++kk) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(sa + kk * kSA + 4 * rg);
    float b[CP];
#pragma unroll
    for (int c = 0; c < CP; ++c) b[c] = sb[kk * l + cg * CP + c];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int c = 0; c < CP; ++c) acc[i][c] = fmaf(a[i], b[c], acc[i][c]);
  }
}

// kTrans = false: part[s][N][l] of E X over K slice s (rows n0 .. n0 + 63).
// kTrans = true:  part[s][K][l] of E^T Y over N slice s (columns k0 .. k0 + 63).
template <bool kTrans, int CP>
__global__ __launch_bounds__(256) void k_lq_mul(const float* __restrict__ E,
                                                const float* __restrict__ Xin, int64_t N,
                                                int64_t K, int64_t slice, float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) float sa[32 * kSA];
  __shared__ __attribute__((aligned(16))) float sb[32 * kLqMaxL];
  constexpr int l = 16 * CP;
  const int tid = threadIdx.x, rg = tid >> 4, cg = tid & 15;
  const int64_t o0 = (int64_t)blockIdx.x * 64;          // first output row
  const int64_t s = blockIdx.y;
  const int64_t rows_out = kTrans ? K : N;
  const int64_t ctot = kTrans ? N : K;                  // contraction length
  const int64_t c0 = s * slice;
  const int64_t c1 = c0 + slice < ctot ? c0 + slice : ctot;
  float acc[4][6] = {};
  // per chunk: 512 float4 of E, 8 CP float4 of the other operand per thread-row
  f32x4 re[2], rx[3];
  auto load = [&](int64_t cb) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int idx = tid + 256 * q;
      if (!kTrans) {  // E rows o0 + row, columns cb + 4 k4
        const int row = idx >> 3, k4 = idx & 7;
        int64_t n = o0 + row;
        if (n >= N) n = N - 1;
        re[q] = *reinterpret_cast<const f32x4*>(E + n * K + cb + 4 * k4);
      } else {        // E rows cb + row (zero past the slice), columns o0 + 4 k4
        const int row = idx >> 4, k4 = idx & 15;
        re[q] = cb + row < c1 ? *reinterpret_cast<const f32x4*>(E + (cb + row) * K + o0 + 4 * k4)
                              : f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      const int idx = tid + 256 * q;  // float4 index within the [32][l] chunk
      if (idx < 8 * l) {
        const int row = idx / (l / 4);
        const bool in = kTrans ? cb + row < c1 : true;
        rx[q] = in ? *reinterpret_cast<const f32x4*>(Xin + cb * l + 4 * idx)
                   : f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int idx = tid + 256 * q;
      if (!kTrans) {  // transpose: sa[kk][row]
        const int row = idx >> 3, k4 = idx & 7;
#pragma unroll
        for (int t = 0; t < 4; ++t) sa[(4 * k4 + t) * kSA + row] = re[q][t];
      } else {
        const int row = idx >> 4, k4 = idx & 15;
        *reinterpret_cast<f32x4*>(sa + row * kSA + 4 * k4) = re[q];
      }
    }
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      const int idx = tid + 256 * q;
      if (idx < 8 * l) *reinterpret_cast<f32x4*>(sb + 4 * idx) = rx[q];
    }
  };
  if (c0 < c1) load(c0);
  for (int64_t cb = c0; cb < c1; cb += 32) {
    __syncthreads();  // the previous chunk's reads are done
    store();
    __syncthreads();
    if (cb + 32 < c1) load(cb + 32);
    chunk_products<CP>(sa, sb, l, rg, cg, acc);
  }
  float* out = part + s * rows_out * l;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t o = o0 + 4 * rg + i;
    if (o >= rows_out) continue;
#pragma unroll
    for (int c = 0; c < CP; ++c) out[o * l + cg * CP + c] = acc[i][c];
  }
}

// out[i] = sum_s part[s][i], s ascending.
template <class T>
__global__ __launch_bounds__(256) void k_lq_reduce(const T* __restrict__ part, int64_t S,
                                                   int64_t count, T* __restrict__ out) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < count;
       i += (int64_t)gridDim.x * blockDim.x) {
    // slices added in order; eight loads issued before their adds, so that
    // they are in flight together (the order, and so the sum, is unchanged)
    T v = part[i];
    int64_t s = 1;
    for (; s + 8 <= S; s += 8) {
      T x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = part[(s + j) * count + i];
#pragma unroll
      for (int j = 0; j < 8; ++j) v += x[j];
    }
    for (; s < S; ++s) v += part[s * count + i];
    out[i] = v;
  }
}

// ---------------------------------------------------------------------------
// partd[s][a][b] = sum over rows t of slice s of X[t][a] X[t][b], in fp64.
// Thread: entries e = tid + 256 m of the l x l matrix.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_lq_gram(const float* __restrict__ X, int64_t T, int l,
                                                 int64_t rows_per_slice,
                                                 double* __restrict__ partd) {
  __shared__ float sx[32 * kLqMaxL];
  constexpr int kMaxE = kLqMaxL * kLqMaxL / 256;
  const int tid = threadIdx.x;
  const int64_t s = blockIdx.x;
  const int64_t tb = s * rows_per_slice;
  const int64_t te = tb + rows_per_slice < T ? tb + rows_per_slice : T;
  const int ll = l * l;
  int ea[kMaxE], eb[kMaxE];
#pragma unroll
  for (int m = 0; m < kMaxE; ++m) {
    const int e = tid + 256 * m;
    ea[m] = e < ll ? e / l : 0;
    eb[m] = e < ll ? e - (e / l) * l : 0;
  }
  double acc[kMaxE] = {};
  for (int64_t c0 = tb; c0 < te; c0 += 32) {
    const int rows = (int)(te - c0 < 32 ? te - c0 : 32);
    for (int e = tid; e < rows * l; e += 256) sx[e] = X[c0 * l + e];
    __syncthreads();
    for (int rr = 0; rr < rows; ++rr) {
#pragma unroll
      for (int m = 0; m < kMaxE; ++m)
        acc[m] = fma((double)sx[rr * l + ea[m]], (double)sx[rr * l + eb[m]], acc[m]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int m = 0; m < kMaxE; ++m) {
    const int e = tid + 256 * m;
    if (e < ll) partd[s * ll + e] = acc[m];
  }
}

// ---------------------------------------------------------------------------
// Eigenvectors of a symmetric l x l matrix G (fp64) by the cyclic Jacobi
// method with a parallel (round-robin) ordering: each round rotates l / 2
// disjoint index pairs at once, l - 1 rounds make a sweep in which every
// pair is rotated once.  A and V live in LDS.  The rotation of pair (p, q)
// zeroes A[p][q] with t = tan(phi) the smaller root of
// t^2 + 2 theta t - 1 = 0, theta = (A[q][q] - A[p][p]) / (2 A[p][q]).
// Sweeps stop when the off-diagonal mass is below 1e-20 of the total (its
// norm below 1e-10, far under the fp32 outputs' rounding) or after 60
// sweeps.  Eigenvalues are then sorted in descending order
// (lam[i]) and the Ritz factors written: M[a][i] = V[a][i_i] lambda_i^{1/4}
// and M[l r + a r + i] = V[a][i_i] lambda_i^{-1/4} for i < r (0 where
// lambda_i <= 0).
// ---------------------------------------------------------------------------
// (t < l - 1 and k < l / 2, so every sum below is under 2 (l - 1): one
// conditional subtraction takes it mod l - 1)
__device__ __forceinline__ void jacobi_pair(int k, int t, int l, int& p, int& q) {
  const int m = l - 1;
  if (k == 0) {
    p = 0;
    q = 1 + t;
  } else {
    int x = t + k, y = t + m - k;
    if (x >= m) x -= m;
    if (y >= m) y -= m;
    p = 1 + x;
    q = 1 + y;
  }
  if (p > q) {
    const int x = p;
    p = q;
    q = x;
  }
}

constexpr int kEigThreads = 1024;

__global__ __launch_bounds__(kEigThreads) void k_lq_eig(const double* __restrict__ G, int l,
                                                        int r, float* __restrict__ M,
                                                        double* __restrict__ lam) {
  extern __shared__ double dsm[];
  // A and V with an odd row stride S (doubles): a column walk (stride S)
  // and a row walk (stride 1) both touch distinct LDS banks across a wave.
  const int S = l | 1;
  double* A = dsm;               // [l][S]
  double* V = dsm + l * S;       // [l][S]
  double* cs = V + l * S;        // [l / 2][2]
  int* pq = reinterpret_cast<int*>(cs + l);  // [l / 2][2]
  __shared__ double red[kEigThreads];
  __shared__ int order[kLqMaxL];
  __shared__ int done;
  const int tid = threadIdx.x;
  const int half = l / 2;
  // thread layout of the rotation phases: pair group kg, 32-lane stripe jl
  const int kg = tid >> 5, jl = tid & 31;
  constexpr int KG = kEigThreads / 32;
  static_assert(2 * KG >= kLqMaxL / 2 && 3 * 32 >= kLqMaxL,
                "a thread's two pairs and three 32-stripes cover every rotation");
  for (int i = kg; i < l; i += KG)
    for (int j = jl; j < l; j += 32) {
      A[i * S + j] = G[i * l + j];
      V[i * S + j] = (i == j) ? 1.0 : 0.0;
    }
  __syncthreads();
  for (int sweep = 0; sweep < 60; ++sweep) {
    // convergence test: off-diagonal mass against the total
    double off = 0.0, tot = 0.0;
    for (int i = kg; i < l; i += KG)
      for (int j = jl; j < l; j += 32) {
        const double v = A[i * S + j] * A[i * S + j];
        tot += v;
        if (i != j) off += v;
      }
    red[tid] = off;
    __syncthreads();
    for (int w = kEigThreads / 2; w > 0; w >>= 1) {
      if (tid < w) red[tid] += red[tid + w];
      __syncthreads();
    }
    const double offs = red[0];
    __syncthreads();
    red[tid] = tot;
    __syncthreads();
    for (int w = kEigThreads / 2; w > 0; w >>= 1) {
      if (tid < w) red[tid] += red[tid + w];
      __syncthreads();
    }
    if (tid == 0) done = !(offs > 1e-20 * red[0]);
    __syncthreads();
    if (done) break;
    for (int t = 0; t < l - 1; ++t) {
      if (tid < half) {
        int p, q;
        jacobi_pair(tid, t, l, p, q);
        const double apq = A[p * S + q];
        double c = 1.0, s = 0.0;
        if (apq != 0.0) {
          // t = sign(theta) / (|theta| + sqrt(theta^2 + 1)) with theta = d / (2 apq),
          // multiplied through by 2 |apq| (one divide instead of two)
          const double d = A[q * S + q] - A[p * S + p];
          const double tt =
              (d >= 0.0 ? 2.0 : -2.0) * apq / (fabs(d) + sqrt(d * d + 4.0 * apq * apq));
          c = rsqrt(tt * tt + 1.0);
          s = tt * c;
        }
        cs[2 * tid] = c;
        cs[2 * tid + 1] = s;
        pq[2 * tid] = p;
        pq[2 * tid + 1] = q;
      }
      __syncthreads();
      // rows p, q of every pair.  Thread (kg, jl) owns pairs kg and kg + KG
      // and columns jl, jl + 32, jl + 64; pairs are disjoint, so all its
      // loads are issued before any of its stores (measured 17 % faster per
      // eigensolve than one load-rotate-store chain at a time).
      {
        double ap[2][3], aq[2][3], c[2], sn[2];
        int p[2], q[2];
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          const int k = kg + KG * a;
          const bool kv = k < half;
          p[a] = kv ? pq[2 * k] : 0;
          q[a] = kv ? pq[2 * k + 1] : 0;
          c[a] = kv ? cs[2 * k] : 1.0;
          sn[a] = kv ? cs[2 * k + 1] : 0.0;
#pragma unroll
          for (int b = 0; b < 3; ++b) {
            const int j = jl + 32 * b;
            if (kv && j < l) {
              ap[a][b] = A[p[a] * S + j];
              aq[a][b] = A[q[a] * S + j];
            }
          }
        }
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int b = 0; b < 3; ++b) {
            const int j = jl + 32 * b;
            if (kg + KG * a < half && j < l) {
              A[p[a] * S + j] = c[a] * ap[a][b] - sn[a] * aq[a][b];
              A[q[a] * S + j] = sn[a] * ap[a][b] + c[a] * aq[a][b];
            }
          }
      }
      __syncthreads();
      // columns p, q of every pair, in A and V (rows jl, jl + 32, jl + 64)
      {
        double ap[2][3], aq[2][3], vp[2][3], vq[2][3], c[2], sn[2];
        int p[2], q[2];
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          const int k = kg + KG * a;
          const bool kv = k < half;
          p[a] = kv ? pq[2 * k] : 0;
          q[a] = kv ? pq[2 * k + 1] : 0;
          c[a] = kv ? cs[2 * k] : 1.0;
          sn[a] = kv ? cs[2 * k + 1] : 0.0;
#pragma unroll
          for (int b = 0; b < 3; ++b) {
            const int i = jl + 32 * b;
            if (kv && i < l) {
              ap[a][b] = A[i * S + p[a]];
              aq[a][b] = A[i * S + q[a]];
              vp[a][b] = V[i * S + p[a]];
              vq[a][b] = V[i * S + q[a]];
            }
          }
        }
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int b = 0; b < 3; ++b) {
            const int i = jl + 32 * b;
            if (kg + KG * a < half && i < l) {
              A[i * S + p[a]] = c[a] * ap[a][b] - sn[a] * aq[a][b];
              A[i * S + q[a]] = sn[a] * ap[a][b] + c[a] * aq[a][b];
              V[i * S + p[a]] = c[a] * vp[a][b] - sn[a] * vq[a][b];
              V[i * S + q[a]] = sn[a] * vp[a][b] + c[a] * vq[a][b];
            }
          }
      }
      __syncthreads();
    }
  }
  // descending order of the eigenvalues (ties keep the lower index first)
  if (tid < l) {
    const double me = A[tid * S + tid];
    int rank = 0;
    for (int j = 0; j < l; ++j) {
      const double o = A[j * S + j];
      rank += (o > me || (o == me && j < tid)) ? 1 : 0;
    }
    order[rank] = tid;
  }
  __syncthreads();
  if (tid < l) lam[tid] = A[order[tid] * S + order[tid]];
  for (int e = tid; e < l * r; e += kEigThreads) {
    const int a = e / r, i = e - a * r;
    const double li = A[order[i] * S + order[i]];
    const double q4 = li > 0.0 ? sqrt(sqrt(li)) : 0.0;
    const double v = V[a * S + order[i]];
    M[e] = (float)(v * q4);
    M[l * r + e] = (float)(q4 > 0.0 ? v / q4 : 0.0);
  }
}

// ---------------------------------------------------------------------------
// Cholesky factor of a Gram matrix G = X^T X (l x l, fp64): G = L L^T, so
// that X L^{-T} has orthonormal columns spanning span(X).  One workgroup,
// right-looking in LDS.  A pivot at or below 1e-10 times the largest
// diagonal of G marks its column as dependent on the earlier ones: the
// column is dropped (left out of the trailing update; its output column
// will be 0), which keeps the other output columns orthonormal.  Writes L
// as fp32 [l][l] (lower; 0 above) and invd[j] = 1 / L[j][j] (0 if dropped).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_lq_chol(const double* __restrict__ G, int l,
                                                 float* __restrict__ Lout,
                                                 float* __restrict__ invd) {
  extern __shared__ double csm[];
  const int S = l | 1;
  double* Lm = csm;  // [l][S]
  __shared__ double dmax;
  const int tid = threadIdx.x, ti = tid >> 5, tk = tid & 31;
  for (int i = ti; i < l; i += 8)
    for (int j = tk; j < l; j += 32) Lm[i * S + j] = G[i * l + j];
  __syncthreads();
  if (tid == 0) {
    double m = 0.0;
    for (int j = 0; j < l; ++j) m = fmax(m, Lm[j * S + j]);
    dmax = m;
  }
  __syncthreads();
  const double tol = kDrop * dmax;
  for (int j = 0; j < l; ++j) {
    const double d = Lm[j * S + j];
    const bool drop = !(d > tol);
    const double piv = drop ? 1.0 : sqrt(d);
    __syncthreads();  // every thread has read the pivot before it changes
    if (tid == 0) {
      Lm[j * S + j] = piv;
      invd[j] = drop ? 0.0f : (float)(1.0 / piv);
    }
    for (int i = j + 1 + tid; i < l; i += 256) Lm[i * S + j] = drop ? 0.0 : Lm[i * S + j] / piv;
    __syncthreads();
    // trailing update of the lower triangle: A[i][k] -= L[i][j] L[k][j], j < k <= i
    for (int i = j + 1 + ti; i < l; i += 8) {
      const double lij = Lm[i * S + j];
      for (int k = j + 1 + tk; k <= i; k += 32) Lm[i * S + k] -= lij * Lm[k * S + j];
    }
    __syncthreads();
  }
  for (int i = ti; i < l; i += 8)
    for (int j = tk; j < l; j += 32) Lout[i * l + j] = j <= i ? (float)Lm[i * S + j] : 0.0f;
}

// out[t] = X[t] L^{-T}: row t of the output solves x L^T = X[t] by forward
// substitution (x_j = (X[t][j] - sum_{k<j} x_k L[j][k]) invd[j]).  One
// thread per row, the row in registers, L broadcast from LDS.
template <int CP>
__global__ __launch_bounds__(256) void k_lq_trsm(const float* __restrict__ X, int64_t T,
                                                 const float* __restrict__ Lf,
                                                 const float* __restrict__ invd,
                                                 float* __restrict__ out) {
  constexpr int l = 16 * CP;
  __shared__ __attribute__((aligned(16))) float sl[l * l];
  __shared__ float sd[l];
  for (int e = threadIdx.x; e < l * l; e += 256) sl[e] = Lf[e];
  if (threadIdx.x < l) sd[threadIdx.x] = invd[threadIdx.x];
  __syncthreads();
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  float x[l];
#pragma unroll
  for (int j = 0; j < l; j += 4) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(X + t * l + j);
    x[j] = v[0]; x[j + 1] = v[1]; x[j + 2] = v[2]; x[j + 3] = v[3];
  }
#pragma unroll
  for (int j = 0; j < l; ++j) {
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
    for (int k = 0; k + 4 <= j; k += 4) {
      const f32x4 lv = *reinterpret_cast<const f32x4*>(sl + j * l + k);
      a0 = fmaf(x[k], lv[0], a0);
      a1 = fmaf(x[k + 1], lv[1], a1);
      a2 = fmaf(x[k + 2], lv[2], a2);
      a3 = fmaf(x[k + 3], lv[3], a3);
    }
#pragma unroll
    for (int k = j & ~3; k < j; ++k) a0 = fmaf(x[k], sl[j * l + k], a0);
    x[j] = (x[j] - ((a0 + a1) + (a2 + a3))) * sd[j];
  }
#pragma unroll
  for (int j = 0; j < l; j += 4)
    *reinterpret_cast<f32x4*>(out + t * l + j) = f32x4{x[j], x[j + 1], x[j + 2], x[j + 3]};
}

// ---------------------------------------------------------------------------
// Y[T][c] = X[T][l] M[l][c] (c <= l).  32 rows per workgroup; thread: row
// tid / 8, columns cg + 8 m.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_lq_mul_xm(const float* __restrict__ X, int64_t T, int l,
                                                   const float* __restrict__ M, int c,
                                                   float* __restrict__ Y) {
  __shared__ float sm[kLqMaxL * kLqMaxL];
  __shared__ float sx[32 * (kLqMaxL + 1)];
  const int tid = threadIdx.x, row = tid >> 3, cg = tid & 7;
  const int64_t t0 = (int64_t)blockIdx.x * 32;
  const int xs = l + 1;
  for (int e = tid; e < l * c; e += 256) sm[e] = M[e];
  for (int e = tid; e < 32 * l; e += 256) {
    const int rr = e / l, j = e - rr * l;
    int64_t t = t0 + rr;
    if (t >= T) t = T - 1;
    sx[rr * xs + j] = X[t * l + j];
  }
  __syncthreads();
  float acc[kLqMaxL / 8] = {};
  const int mc = (c + 7 - cg) / 8;  // columns cg, cg + 8, ... below c
  for (int j = 0; j < l; ++j) {
    const float x = sx[row * xs + j];
#pragma unroll
    for (int m = 0; m < kLqMaxL / 8; ++m)
      if (m < mc) acc[m] = fmaf(x, sm[j * c + cg + 8 * m], acc[m]);
  }
  const int64_t t = t0 + row;
  if (t < T) {
#pragma unroll
    for (int m = 0; m < kLqMaxL / 8; ++m)
      if (m < mc) Y[t * c + cg + 8 * m] = acc[m];
  }
}

// A[i][k] = bf16(L2t[k][i]); B[n][i] = bf16(L1[n][i] / s).
__global__ __launch_bounds__(256) void k_lq_adapter(const float* __restrict__ L1,
                                                    const float* __restrict__ L2t, int64_t N,
                                                    int64_t K, int r, float s,
                                                    uint16_t* __restrict__ A,
                                                    uint16_t* __restrict__ B) {
  const int64_t na = (int64_t)r * K, total = na + N * r;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    if (e < na) {
      const int64_t i = e / K, k = e - i * K;
      A[e] = f32_to_bf16(L2t[k * r + i]);
    } else {
      const int64_t f = e - na;
      B[f] = f32_to_bf16(L1[f] / s);
    }
  }
}

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// f(std::integral_constant<int, cp>) for cp = l / 16 in 1 .. 6
template <class F>
void with_cp(int cp, F&& f) {
  switch (cp) {
    case 1: f(std::integral_constant<int, 1>{}); break;
    case 2: f(std::integral_constant<int, 2>{}); break;
    case 3: f(std::integral_constant<int, 3>{}); break;
    case 4: f(std::integral_constant<int, 4>{}); break;
    case 5: f(std::integral_constant<int, 5>{}); break;
    default: f(std::integral_constant<int, 6>{}); break;
  }
}
inline size_t al(size_t v) { return (v + 255) / 256 * 256; }

// Contraction slices of the two E products (multiples of 32 long): enough
// workgroups (64 output rows each) to fill the chip twice.
inline int64_t mul_slice_len(int64_t rows_out, int64_t ctot) {
  const int64_t tiles = cdiv(rows_out, 64);
  int64_t ns = cdiv(512, tiles);
  if (ns > cdiv(ctot, 256)) ns = cdiv(ctot, 256);  // at least 256 deep
  if (ns < 1) ns = 1;
  return cdiv(cdiv(ctot, ns), 32) * 32;
}
inline int64_t mul_slices(int64_t rows_out, int64_t ctot) {
  return cdiv(ctot, mul_slice_len(rows_out, ctot));
}
inline int64_t gram_slices(int64_t T) {
  int64_t s = cdiv(T, 32);
  if (s > 512) s = 512;
  return s < 1 ? 1 : s;
}

struct LqPlan {
  size_t e_off, y_off, y2_off, z_off, z2_off, part_off, partd_off, g_off, m_off, lam_off, total;
};

LqPlan plan(int64_t N, int64_t K, int l) {
  LqPlan p{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += al(bytes);
    return at;
  };
  p.e_off = take(4 * (size_t)N * K);
  p.y_off = take(4 * (size_t)N * l);
  p.y2_off = take(4 * (size_t)N * l);
  p.z_off = take(4 * (size_t)K * l);
  p.z2_off = take(4 * (size_t)K * l);
  const int64_t sx = mul_slices(N, K), sy = mul_slices(K, N);
  p.part_off = take(4 * (size_t)(sx * N > sy * K ? sx * N : sy * K) * l);
  const int64_t gs = gram_slices(N > K ? N : K);
  p.partd_off = take(8 * (size_t)gs * l * l);
  p.g_off = take(8 * (size_t)l * l);
  p.m_off = take(4 * (size_t)2 * l * l);
  p.lam_off = take(8 * (size_t)l);
  p.total = o;
  return p;
}

size_t eig_lds(int l) { return (size_t)(2 * l * (l | 1) + l) * 8 + (size_t)l * 4; }
size_t chol_lds(int l) { return (size_t)(l * (l | 1)) * 8; }

}  // namespace

size_t lq_workspace_bytes(int64_t N, int64_t K, int32_t l) { return plan(N, K, l).total; }

hipError_t launch_lq_residual(const float* W, const float* L1, const float* L2t, int64_t N,
                              int64_t K, int r, float* R, hipStream_t stream) {
  hipLaunchKernelGGL(k_lq_residual, dim3((unsigned)(cdiv(N, 64) * (K / 64))), dim3(256), 0, stream,
                     W, L1, L2t, N, K, r, R);
  return hipGetLastError();
}

hipError_t launch_lq_init(const LqArgs& a, hipStream_t stream) {
  // The two one-workgroup solvers use more than the default 64 KB of
  // dynamic LDS; the limit is raised on every call (cheap, idempotent), so
  // that it holds for whichever device is current.
  hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_lq_eig),
                                        hipFuncAttributeMaxDynamicSharedMemorySize,
                                        (int)eig_lds(kLqMaxL));
  if (attr == hipSuccess)
    attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_lq_chol),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)chol_lds(kLqMaxL));
  if (attr != hipSuccess) return attr;
  const int64_t N = a.N, K = a.K;
  const int l = a.l, r = a.r;
  const LqPlan pl = plan(N, K, l);
  char* base = static_cast<char*>(a.ws);
  float* ebuf = reinterpret_cast<float*>(base + pl.e_off);
  float* Y = reinterpret_cast<float*>(base + pl.y_off);
  float* Y2 = reinterpret_cast<float*>(base + pl.y2_off);
  float* Z = reinterpret_cast<float*>(base + pl.z_off);
  float* Z2 = reinterpret_cast<float*>(base + pl.z2_off);
  float* part = reinterpret_cast<float*>(base + pl.part_off);
  double* partd = reinterpret_cast<double*>(base + pl.partd_off);
  double* G = reinterpret_cast<double*>(base + pl.g_off);
  float* Mm = reinterpret_cast<float*>(base + pl.m_off);
  double* lam = reinterpret_cast<double*>(base + pl.lam_off);
  const int64_t nblocks = N * K / 64;

  hipError_t e = hipSuccess;
  auto ok = [&]() { return (e = hipGetLastError()) == hipSuccess; };

  // one of the two E products into out, through the partial buffer
  auto mul = [&](bool trans, const float* E, const float* X, float* out) {
    const int64_t rows_out = trans ? K : N, ctot = trans ? N : K;
    const int64_t len = mul_slice_len(rows_out, ctot), S = cdiv(ctot, len);
    const dim3 grid((unsigned)cdiv(rows_out, 64), (unsigned)S);
    const int cp = l / 16;
    with_cp(cp, [&](auto cpc) {
      constexpr int CP = decltype(cpc)::value;
      if (trans)
        hipLaunchKernelGGL((k_lq_mul<true, CP>), grid, dim3(256), 0, stream, E, X, N, K, len, part);
      else
        hipLaunchKernelGGL((k_lq_mul<false, CP>), grid, dim3(256), 0, stream, E, X, N, K, len, part);
    });
    if (!ok()) return false;
    hipLaunchKernelGGL(k_lq_reduce<float>, dim3((unsigned)cdiv(rows_out * l, 256)), dim3(256), 0,
                       stream, part, S, rows_out * l, out);
    return ok();
  };
  auto mul_ex = [&](const float* E, const float* X, float* out) { return mul(false, E, X, out); };
  auto mul_ety = [&](const float* E, const float* Y, float* out) { return mul(true, E, Y, out); };
  auto gram = [&](const float* X, int64_t T) {
    const int64_t S = gram_slices(T), rps = cdiv(T, S);
    hipLaunchKernelGGL(k_lq_gram, dim3((unsigned)cdiv(T, rps)), dim3(256), 0, stream, X, T, l, rps,
                       partd);
    if (!ok()) return false;
    hipLaunchKernelGGL(k_lq_reduce<double>, dim3((unsigned)cdiv((int64_t)l * l, 256)), dim3(256), 0,
                       stream, partd, cdiv(T, rps), (int64_t)l * l, G);
    return ok();
  };
  auto ritz_factors = [&](const float* X, int64_t T) {
    if (!gram(X, T)) return false;
    hipLaunchKernelGGL(k_lq_eig, dim3(1), dim3(kEigThreads), eig_lds(l), stream, G, l, r, Mm, lam);
    return ok();
  };
  auto mul_xm = [&](const float* X, int64_t T, const float* M, int c, float* out) {
    hipLaunchKernelGGL(k_lq_mul_xm, dim3((unsigned)cdiv(T, 32)), dim3(256), 0, stream, X, T, l, M,
                       c, out);
    return ok();
  };
  // orthonormalize X [T][l] into out (a different buffer)
  auto orth = [&](const float* X, int64_t T, float* out) {
    if (!gram(X, T)) return false;
    float* invd = Mm + (size_t)l * l;
    hipLaunchKernelGGL(k_lq_chol, dim3(1), dim3(256), chol_lds(l), stream, G, l, Mm, invd);
    if (!ok()) return false;
    with_cp(l / 16, [&](auto cpc) {
      constexpr int CP = decltype(cpc)::value;
      hipLaunchKernelGGL((k_lq_trsm<CP>), dim3((unsigned)cdiv(T, 256)), dim3(256), 0, stream, X, T,
                         Mm, invd, out);
    });
    return ok();
  };
  // L step on E: L1 [N][r], L2t [K][r]
  auto l_step = [&](const float* E) {
    if (!mul_ex(E, a.omega, Y)) return false;
    for (int it = 0; it < a.power_iters; ++it) {
      if (!orth(Y, N, Y2)) return false;       // Y2 = orth(Y)
      if (!mul_ety(E, Y2, Z)) return false;    // Z = E^T Y2
      if (!orth(Z, K, Z2)) return false;       // Z2 = orth(Z)
      if (!mul_ex(E, Z2, Y)) return false;     // Y = E Z2
    }
    if (!orth(Y, N, Y2)) return false;         // Y2 = orth(Y)
    if (!mul_ety(E, Y2, Z)) return false;      // Z = E^T Y2 = B^T
    if (!ritz_factors(Z, K)) return false;     // Ritz factors
    return mul_xm(Y2, N, Mm, r, a.L1) && mul_xm(Z, K, Mm + (size_t)l * r, r, a.L2t);
  };
  auto q_step = [&](const float* R) {
    return (e = launch_nf4_quantize(R, nblocks, a.codes, a.q8, a.step, a.code, 0, nullptr, stream)) ==
           hipSuccess;
  };
  auto residual = [&]() {
    hipLaunchKernelGGL(k_lq_residual, dim3((unsigned)(cdiv(N, 64) * (K / 64))), dim3(256), 0,
                       stream, a.W, a.L1, a.L2t, N, K, r, ebuf);
    return ok();
  };
  auto error = [&]() {
    const int64_t n8 = N * K / 8;
    int64_t grid = cdiv(n8, 256);
    if (grid > 65536) grid = 65536;
    return with_code(a.code, [&](auto ct) {
      hipLaunchKernelGGL(k_lq_error<decltype(ct)>, dim3((unsigned)grid), dim3(256), 0, stream,
                         a.W, a.codes, a.q8, a.step, n8, ebuf);
      return ok();
    });
  };

  for (int it = 0; it < a.iters; ++it) {
    if (a.start == 0) {  // L step, then Q step
      const float* E = a.W;
      if (it > 0) {
        if (!error()) return e;
        E = ebuf;
      }
      if (!l_step(E) || !residual() || !q_step(ebuf)) return e;
    } else {  // Q step, then L step
      if (it == 0) {
        if (!q_step(a.W)) return e;
      } else if (!residual() || !q_step(ebuf)) {
        return e;
      }
      if (!error() || !l_step(ebuf)) return e;
    }
  }
  const int64_t tot = (int64_t)r * K + N * r;
  int64_t grid = cdiv(tot, 256);
  if (grid > 65536) grid = 65536;
  hipLaunchKernelGGL(k_lq_adapter, dim3((unsigned)grid), dim3(256), 0, stream, a.L1, a.L2t, N, K,
                     r, a.s, a.A, a.B);
  ok();
  return e;
}

}  // namespace qn
