// Internal launch interface between the C ABI (abi.hip) and the kernels.
// Every launcher enqueues on `stream` and returns hipGetLastError().
#pragma once

#include "common.hpp"

namespace qn {

// ---- nf4_quant.hip ----  (code: kId of any code type; ut: the caller's
// codebook for the CodeUser types, else unused and may be null)
// Blocks of 64 << bshift elements (bshift 0, 1, 2: block size 64, 128, 256);
// nblocks counts those blocks.
hipError_t launch_nf4_quantize(const float* W, int64_t nblocks, uint8_t* codes, uint8_t* q8,
                               float* step, int code, int bshift, const UserTable* ut,
                               hipStream_t stream);
hipError_t launch_nf4_dequantize(const uint8_t* codes, const uint8_t* q8, const float* step,
                                 int64_t nelem, uint16_t* out, int code, int bshift,
                                 const UserTable* ut, hipStream_t stream);

// ---- qgemm.hip: MFMA tile kernels with the NF4 dequantization in the prologue ----
struct Nf4View {
  const uint8_t* codes;
  const uint8_t* q8;
  const float* step;
  int64_t N, K;
  int code;     // kId of the code type
  int bshift;   // block size 64 << bshift (K is a multiple of it)
  UserTable ut; // the caller's codebook (CodeUser types only)
};

// Y[M,N] = X[M,K] W^T + bf16(s U)[M,r] B[N,r]^T.  U has row stride ldu (a
// multiple of 8, zero-padded to ceil(r/64)*64 columns).
hipError_t launch_qgemm_fwd(const Nf4View& w, const uint16_t* X, int64_t M, const uint16_t* U,
                            int64_t ldu, const uint16_t* B, int32_t r, float s, uint16_t* Y,
                            hipStream_t stream);

// dX[M,K] = dY[M,N] W + dU[M,r] A[r,K].  dU has row stride lddu (zero-padded).
hipError_t launch_qgemm_bwd(const Nf4View& w, const uint16_t* dY, int64_t M, const uint16_t* dU,
                            int64_t lddu, const uint16_t* A, int32_t r, uint16_t* dX,
                            hipStream_t stream);

// ---- gemv.hip: bandwidth-bound forward for M <= 16 ----
constexpr int kGemvMaxM = 16;
// Whether launch_qgemv takes these sizes (its per-workgroup table of block
// constants must fit in LDS: K up to about 32000 at 16 tokens and rank 256).
bool gemv_fits(int64_t M, int32_t r, int64_t K);
// Workspace of launch_qgemv: fp32 partial sums of U = X A^T.
size_t gemv_workspace_bytes(int64_t M, int32_t r, int64_t K);
// Y = X W^T + s (X A^T) B^T for M <= kGemvMaxM, and bf16 U into U_out when
// it is not null.  Two launches (U partial sums, then the weight stream);
// ev0 / ev1 (nullable) are recorded around the second one.
hipError_t launch_qgemv(const Nf4View& w, const uint16_t* X, int64_t M, const uint16_t* A,
                        const uint16_t* B, int32_t r, float s, uint16_t* Y, uint16_t* U_out,
                        float* upart, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1);

// ---- lora.hip: small-rank products with in-kernel reduction of contraction slices ----
// Operand element access: A-op (i, c) at a[i*a_si + c*a_sc]; B-op (c, j) at
// b[j*b_sj + c*b_sc]; one stride of each operand must be 1.
struct SkinnyOp {
  const uint16_t* a;
  int64_t a_si, a_sc;
  const uint16_t* b;
  int64_t b_sj, b_sc;
  int64_t I, J, C;
};
// One product: out[i*o_si + j] = bf16(scale * sum_c Aop(i,c) Bop(c,j)) for
// j < J, zero for J <= j < Jw, optionally also out2[i*o2_si + j] for j < J.
// part: fp32 slice partials (size from skinny_partial_bytes; unused when the
// product has one slice).
struct SkinnyJob {
  SkinnyOp op;
  float scale;
  uint16_t* out;
  int64_t o_si, Jw;
  uint16_t* out2;
  int64_t o2_si;
  float* part;
};
int skinny_tiles(int64_t I, int64_t J);
int skinny_splits(int64_t I, int64_t J, int64_t C);
size_t skinny_partial_bytes(int64_t I, int64_t J, int64_t C);
SkinnyJob make_job(const SkinnyOp& op, float scale, uint16_t* out, int64_t o_si, int64_t Jw,
                   uint16_t* out2, int64_t o2_si, float* part);
// Run one or two independent products: one launch for the partial products
// and, if any product has several contraction slices, one finish launch.
hipError_t launch_skinny(const SkinnyJob* jobs, int njobs, hipStream_t stream);

// ---- lq_init.hip: low-rank plus quantized decomposition of a weight ----
struct LqArgs {
  const float* W;      // [N, K]
  int64_t N, K;
  int code;            // code type id of the Q component
  int r, l;            // rank, subspace width (r < l <= 96, l % 16 == 0)
  const float* omega;  // [K, l] Gaussian test matrix
  int iters, power_iters;
  int start;           // 0: L step first (Q = 0), 1: Q step first (L = 0)
  float s;             // LoRA scale of the adapter outputs
  uint8_t* codes;
  uint8_t* q8;
  float* step;
  uint16_t* A;         // [r, K] bf16
  uint16_t* B;         // [N, r] bf16
  float* L1;           // [N, r]
  float* L2t;          // [K, r]
  void* ws;            // lq_workspace_bytes(N, K, l) bytes, 256-byte aligned
};
size_t lq_workspace_bytes(int64_t N, int64_t K, int32_t l);
hipError_t launch_lq_init(const LqArgs& a, hipStream_t stream);
// R = W - L1 L2t^T (fp32 [N, K]; L1 [N, r], L2t [K, r], r <= 96, K % 64 == 0)
hipError_t launch_lq_residual(const float* W, const float* L1, const float* L2t, int64_t N,
                              int64_t K, int r, float* R, hipStream_t stream);

// ---- stream.hip: read-only HBM stream (measurement helper) ----
// Reads bytes / 16 16-byte words of src with `grid` workgroups of 256
// lanes; writes one word per workgroup to sink[0 .. grid - 1].
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int grid,
                              hipStream_t stream);

// ---- ilp.hip: configuration errors and the budget program ----
size_t quant_error_workspace_bytes(int64_t N, int64_t K, int bits, int bshift, bool lowrank);
// *sq_err (device) = ||R - W_hat(R)||_F^2, R = W or W - L1 L2t^T (L1 non-null)
hipError_t launch_quant_error(const float* W, int64_t N, int64_t K, int code, int bshift,
                              const float* L1, const float* L2t, int r, double* sq_err, void* ws,
                              hipStream_t stream);
// host: exact minimum-error choice within the budget; false if none fits
bool ilp_plan(int M, int C, const double* err, const int64_t* bytes, int64_t budget,
              int32_t* choice, double* total_err, int64_t* total_bytes);

}  // namespace qn
