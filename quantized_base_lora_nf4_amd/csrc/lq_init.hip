// Low-rank plus quantized decomposition of a frozen weight, W ~ Q + L1 L2
// ("LQ-LoRA: Low-rank Plus Quantized Matrix Decomposition for Efficient
// Language Model Finetuning", abstract: an iterative algorithm splits each
// pretrained matrix into a high-precision low-rank component, trained as the
// adapter, and a fixed quantized component).
//
// Alternating minimization of ||W - Q - L1 L2||_F:
//   L step  rank-r approximation of E = W - Q: randomized subspace iteration
//           from the caller's Gaussian test matrix Omega [K, l] (Halko,
//           Martinsson and Tropp 2011, algorithm 4.4), then Rayleigh-Ritz on
//           the l-dimensional subspace;
//   Q step  the block quantizer (nf4_quant.hip) on R = W - L1 L2.
//
// Kernels (all fp32 data, fp64 for the l x l Gram matrices and their
// eigenvectors):
//   k_lq_residual   R = W - L1 L2t^T                    (tiles, HBM + VALU)
//   k_lq_error      E = W - W_hat(Q)                    (elementwise, HBM)
//   k_lq_mul_ex     Y = E X      [N,K] x [K,l]          (E streamed once)
//   k_lq_mul_ety    partial Z = E^T Y over row slices   (E streamed once)
//   k_lq_reduce     sum of the slices, fixed order
//   k_lq_gram       partial X^T X over row slices, fp64
//   k_lq_eig        Jacobi eigenvectors of an l x l matrix, one workgroup
//   k_lq_mul_xm     Y = X M      [T,l] x [l,c]
//   k_lq_adapter    A = bf16(L2), B = bf16(L1 / s)
// No atomics: every sum has a fixed order, so results are reproducible.
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
// Y[N,l] = E[N,K] X[K,l].  32 rows per workgroup; thread: rows ty, ty + 16,
// columns cg + 16 m (m < l / 16).  K in chunks of 32 through LDS.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_lq_mul_ex(const float* __restrict__ E,
                                                   const float* __restrict__ X, int64_t N,
                                                   int64_t K, int l, float* __restrict__ Y) {
  __shared__ float se[32 * 33];
  __shared__ float sx[32 * kLqMaxL];
  const int tid = threadIdx.x, cg = tid & 15, ty = tid >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * 32;
  const int mc = l >> 4;
  float acc[2][kLqMaxL / 16] = {};
  for (int64_t k0 = 0; k0 < K; k0 += 32) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = tid + 256 * q, row = e >> 5, col = e & 31;
      int64_t n = n0 + row;
      if (n >= N) n = N - 1;
      se[row * 33 + col] = E[n * K + k0 + col];
    }
    for (int e = tid; e < 32 * l; e += 256) sx[e] = X[k0 * l + e];
    __syncthreads();
#pragma unroll 4
    for (int kk = 0; kk < 32; ++kk) {
      const float e0 = se[ty * 33 + kk], e1 = se[(ty + 16) * 33 + kk];
#pragma unroll
      for (int m = 0; m < kLqMaxL / 16; ++m) {
        if (m < mc) {
          const float x = sx[kk * l + cg + 16 * m];
          acc[0][m] = fmaf(e0, x, acc[0][m]);
          acc[1][m] = fmaf(e1, x, acc[1][m]);
        }
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int64_t n = n0 + ty + 16 * h;
    if (n >= N) continue;
#pragma unroll
    for (int m = 0; m < kLqMaxL / 16; ++m)
      if (m < mc) Y[n * l + cg + 16 * m] = acc[h][m];
  }
}

// ---------------------------------------------------------------------------
// part[s][K][l] = sum over rows n of slice s of E[n][k] Y[n][j].  Workgroup:
// 64 columns of E and one slice of rows; thread: column kk, output columns
// jg + 4 m (m < l / 4).  Rows in chunks of 32 through LDS.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_lq_mul_ety(const float* __restrict__ E,
                                                    const float* __restrict__ Y, int64_t N,
                                                    int64_t K, int l, int64_t rows_per_slice,
                                                    float* __restrict__ part) {
  __shared__ float se[32 * 64];
  __shared__ float sy[32 * kLqMaxL];
  const int tid = threadIdx.x, kk = tid & 63, jg = tid >> 6;
  const int64_t k0 = (int64_t)blockIdx.x * 64;
  const int64_t s = blockIdx.y;
  const int64_t nb = s * rows_per_slice;
  const int64_t ne = nb + rows_per_slice < N ? nb + rows_per_slice : N;
  const int mc = l >> 2;
  float acc[kLqMaxL / 4] = {};
  for (int64_t c0 = nb; c0 < ne; c0 += 32) {
    const int rows = (int)(ne - c0 < 32 ? ne - c0 : 32);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int e = tid + 256 * q, row = e >> 6, col = e & 63;
      se[e] = row < rows ? E[(c0 + row) * K + k0 + col] : 0.0f;
    }
    for (int e = tid; e < 32 * l; e += 256) {
      const int row = e / l;
      sy[e] = row < rows ? Y[c0 * l + e] : 0.0f;
    }
    __syncthreads();
    for (int rr = 0; rr < rows; ++rr) {
      const float ev = se[rr * 64 + kk];
#pragma unroll
      for (int m = 0; m < kLqMaxL / 4; ++m)
        if (m < mc) acc[m] = fmaf(ev, sy[rr * l + jg + 4 * m], acc[m]);
    }
    __syncthreads();
  }
  float* out = part + (s * K + k0 + kk) * l;
#pragma unroll
  for (int m = 0; m < kLqMaxL / 4; ++m)
    if (m < mc) out[jg + 4 * m] = acc[m];
}

// out[i] = sum_s part[s][i], s ascending.
template <class T>
__global__ __launch_bounds__(256) void k_lq_reduce(const T* __restrict__ part, int64_t S,
                                                   int64_t count, T* __restrict__ out) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < count;
       i += (int64_t)gridDim.x * blockDim.x) {
    T v = part[i];
    for (int64_t s = 1; s < S; ++s) v += part[s * count + i];
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
// Sweeps stop when the off-diagonal mass is below 1e-28 of the total (or
// after 60 sweeps).  Eigenvalues are then sorted in descending order and:
//   mode 0 (orthonormalizer)  M[a][b] = V[a][i_b] lambda_b^{-1/2}, l x l,
//                             0 where lambda_b <= 1e-10 lambda_max;
//   mode 1 (Ritz factors)     M[a][i] = V[a][i_i] lambda_i^{1/4} and
//                             M[l r + a r + i] = V[a][i_i] lambda_i^{-1/4},
//                             i < r (0 where lambda_i <= 0).
// lam[i] receives the sorted eigenvalues.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void jacobi_pair(int k, int t, int l, int& p, int& q) {
  const int m = l - 1;
  if (k == 0) {
    p = 0;
    q = 1 + t % m;
  } else {
    p = 1 + (t + k) % m;
    q = 1 + (t + m - k) % m;
  }
  if (p > q) {
    const int x = p;
    p = q;
    q = x;
  }
}

__global__ __launch_bounds__(256) void k_lq_eig(const double* __restrict__ G, int l, int r,
                                                int mode, float* __restrict__ M,
                                                double* __restrict__ lam) {
  extern __shared__ double dsm[];
  double* A = dsm;               // [l][l]
  double* V = dsm + l * l;       // [l][l]
  double* cs = V + l * l;        // [l / 2][2]
  int* pq = reinterpret_cast<int*>(cs + l);  // [l / 2][2]
  __shared__ double red[256];
  __shared__ int order[kLqMaxL];
  __shared__ int done;
  const int tid = threadIdx.x;
  const int ll = l * l, half = l / 2;
  for (int e = tid; e < ll; e += 256) {
    A[e] = G[e];
    V[e] = (e / l == e % l) ? 1.0 : 0.0;
  }
  __syncthreads();
  for (int sweep = 0; sweep < 60; ++sweep) {
    // convergence test: off-diagonal mass against the total
    double off = 0.0, tot = 0.0;
    for (int e = tid; e < ll; e += 256) {
      const double v = A[e] * A[e];
      tot += v;
      if (e / l != e % l) off += v;
    }
    red[tid] = off;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
      if (tid < w) red[tid] += red[tid + w];
      __syncthreads();
    }
    const double offs = red[0];
    __syncthreads();
    red[tid] = tot;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
      if (tid < w) red[tid] += red[tid + w];
      __syncthreads();
    }
    if (tid == 0) done = !(offs > 1e-28 * red[0]);
    __syncthreads();
    if (done) break;
    for (int t = 0; t < l - 1; ++t) {
      if (tid < half) {
        int p, q;
        jacobi_pair(tid, t, l, p, q);
        const double apq = A[p * l + q];
        double c = 1.0, s = 0.0;
        if (apq != 0.0) {
          const double theta = (A[q * l + q] - A[p * l + p]) / (2.0 * apq);
          const double tt = (theta >= 0.0 ? 1.0 : -1.0) / (fabs(theta) + sqrt(theta * theta + 1.0));
          c = 1.0 / sqrt(tt * tt + 1.0);
          s = tt * c;
        }
        cs[2 * tid] = c;
        cs[2 * tid + 1] = s;
        pq[2 * tid] = p;
        pq[2 * tid + 1] = q;
      }
      __syncthreads();
      // rows p, q of every pair
      for (int e = tid; e < half * l; e += 256) {
        const int k = e / l, j = e - k * l;
        const int p = pq[2 * k], q = pq[2 * k + 1];
        const double c = cs[2 * k], s = cs[2 * k + 1];
        const double ap = A[p * l + j], aq = A[q * l + j];
        A[p * l + j] = c * ap - s * aq;
        A[q * l + j] = s * ap + c * aq;
      }
      __syncthreads();
      // columns p, q of every pair, in A and V
      for (int e = tid; e < half * l; e += 256) {
        const int k = e / l, i = e - k * l;
        const int p = pq[2 * k], q = pq[2 * k + 1];
        const double c = cs[2 * k], s = cs[2 * k + 1];
        const double ap = A[i * l + p], aq = A[i * l + q];
        A[i * l + p] = c * ap - s * aq;
        A[i * l + q] = s * ap + c * aq;
        const double vp = V[i * l + p], vq = V[i * l + q];
        V[i * l + p] = c * vp - s * vq;
        V[i * l + q] = s * vp + c * vq;
      }
      __syncthreads();
    }
  }
  // descending order of the eigenvalues (ties keep the lower index first)
  if (tid < l) {
    const double me = A[tid * l + tid];
    int rank = 0;
    for (int j = 0; j < l; ++j) {
      const double o = A[j * l + j];
      rank += (o > me || (o == me && j < tid)) ? 1 : 0;
    }
    order[rank] = tid;
  }
  __syncthreads();
  if (tid < l) lam[tid] = A[order[tid] * l + order[tid]];
  const double lmax = A[order[0] * l + order[0]];
  if (mode == 0) {
    for (int e = tid; e < ll; e += 256) {
      const int a = e / l, b = e - a * l;
      const double lb = A[order[b] * l + order[b]];
      const double sc = lb > kDrop * lmax ? 1.0 / sqrt(lb) : 0.0;
      M[e] = (float)(V[a * l + order[b]] * sc);
    }
  } else {
    for (int e = tid; e < l * r; e += 256) {
      const int a = e / r, i = e - a * r;
      const double li = A[order[i] * l + order[i]];
      const double q4 = li > 0.0 ? sqrt(sqrt(li)) : 0.0;
      const double v = V[a * l + order[i]];
      M[e] = (float)(v * q4);
      M[l * r + e] = (float)(q4 > 0.0 ? v / q4 : 0.0);
    }
  }
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
inline size_t al(size_t v) { return (v + 255) / 256 * 256; }

// Slices of the E^T Y product: enough workgroups to fill the chip.
inline int64_t ety_slices(int64_t N, int64_t K) {
  int64_t s = cdiv(512, K / 64);
  const int64_t cap = cdiv(N, 32);
  if (s > cap) s = cap;
  return s < 1 ? 1 : s;
}
inline int64_t gram_slices(int64_t T) {
  int64_t s = cdiv(T, 256);
  if (s > 128) s = 128;
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
  p.part_off = take(4 * (size_t)ety_slices(N, K) * K * l);
  const int64_t gs = gram_slices(N > K ? N : K);
  p.partd_off = take(8 * (size_t)gs * l * l);
  p.g_off = take(8 * (size_t)l * l);
  p.m_off = take(4 * (size_t)2 * l * l);
  p.lam_off = take(8 * (size_t)l);
  p.total = o;
  return p;
}

size_t eig_lds(int l) { return (size_t)(2 * l * l + l) * 8 + (size_t)l * 4; }

}  // namespace

size_t lq_workspace_bytes(int64_t N, int64_t K, int32_t l) { return plan(N, K, l).total; }

hipError_t launch_lq_init(const LqArgs& a, hipStream_t stream) {
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&k_lq_eig), hipFuncAttributeMaxDynamicSharedMemorySize,
      (int)eig_lds(kLqMaxL));
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

  auto mul_ex = [&](const float* E, const float* X, float* out) {
    hipLaunchKernelGGL(k_lq_mul_ex, dim3((unsigned)cdiv(N, 32)), dim3(256), 0, stream, E, X, N,
                       K, l, out);
    return ok();
  };
  auto mul_ety = [&](const float* E, const float* Yin, float* out) {
    const int64_t S = ety_slices(N, K), rps = cdiv(N, S);
    hipLaunchKernelGGL(k_lq_mul_ety, dim3((unsigned)(K / 64), (unsigned)S), dim3(256), 0, stream,
                       E, Yin, N, K, l, rps, part);
    if (!ok()) return false;
    hipLaunchKernelGGL(k_lq_reduce<float>, dim3((unsigned)cdiv(K * l, 256)), dim3(256), 0, stream,
                       part, S, K * l, out);
    return ok();
  };
  auto gram_eig = [&](const float* X, int64_t T, int mode) {
    const int64_t S = gram_slices(T), rps = cdiv(T, S);
    hipLaunchKernelGGL(k_lq_gram, dim3((unsigned)S), dim3(256), 0, stream, X, T, l, rps, partd);
    if (!ok()) return false;
    hipLaunchKernelGGL(k_lq_reduce<double>, dim3((unsigned)cdiv((int64_t)l * l, 256)), dim3(256), 0,
                       stream, partd, S, (int64_t)l * l, G);
    if (!ok()) return false;
    hipLaunchKernelGGL(k_lq_eig, dim3(1), dim3(256), eig_lds(l), stream, G, l, r, mode, Mm, lam);
    return ok();
  };
  auto mul_xm = [&](const float* X, int64_t T, const float* M, int c, float* out) {
    hipLaunchKernelGGL(k_lq_mul_xm, dim3((unsigned)cdiv(T, 32)), dim3(256), 0, stream, X, T, l, M,
                       c, out);
    return ok();
  };
  // orthonormalize X [T][l] into out (a different buffer)
  auto orth = [&](const float* X, int64_t T, float* out) {
    return gram_eig(X, T, 0) && mul_xm(X, T, Mm, l, out);
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
    if (!gram_eig(Z, K, 1)) return false;      // Ritz factors
    return mul_xm(Y2, N, Mm, r, a.L1) && mul_xm(Z, K, Mm + (size_t)l * r, r, a.L2t);
  };
  auto q_step = [&](const float* R) {
    return (e = launch_nf4_quantize(R, nblocks, a.codes, a.q8, a.step, a.code, stream)) ==
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
