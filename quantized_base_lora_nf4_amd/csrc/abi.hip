// C ABI of the NF4 + LoRA linear layer: argument checks, workspace carving
// and the launch sequence of each call.  The declarations, with the meaning,
// layout and ownership of every argument, are in include/qlora_nf4.h.
#include "../../include/qlora_nf4.h"

#include <math.h>

#include "kernels.hpp"

using namespace qn;

namespace {

constexpr size_t kAlign = 256;

inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
inline int64_t rank_pad(int32_t r) { return ((int64_t)r + 63) / 64 * 64; }

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct FwdPlan {
  size_t u_off, part_off, total;
  int u_splits;
  int gemv_splits_n;
};

struct BwdPlan {
  size_t u_off, du_off, part_off, total;
};

bool sizes_ok(int64_t M, int64_t N, int64_t K, int32_t r) {
  return M >= 1 && N >= 1 && K >= 64 && (K % 64) == 0 && (N % 8) == 0 && r >= 1 &&
         r <= QLORA_MAX_RANK && M <= ((int64_t)1 << 31) && N <= ((int64_t)1 << 31) &&
         K <= ((int64_t)1 << 31);
}

FwdPlan plan_fwd(int64_t M, int64_t N, int64_t K, int32_t r) {
  FwdPlan p{};
  const int64_t rp = rank_pad(r);
  p.u_off = 0;
  size_t off = align_up((size_t)M * rp * 2);
  p.part_off = off;
  size_t part = skinny_partial_bytes(M, r, K);
  p.u_splits = skinny_splits(M, r, K);
  p.gemv_splits_n = 0;
  if (M <= kGemvMaxM) {
    p.gemv_splits_n = gemv_splits(N, K);
    const size_t g = (size_t)p.gemv_splits_n * M * N * sizeof(float);
    if (g > part) part = g;
  }
  p.total = off + align_up(part);
  return p;
}

BwdPlan plan_bwd(int64_t M, int64_t N, int64_t K, int32_t r) {
  BwdPlan p{};
  const int64_t rp = rank_pad(r);
  p.u_off = 0;
  p.du_off = align_up((size_t)M * rp * 2);
  p.part_off = p.du_off + align_up((size_t)M * rp * 2);
  size_t part = skinny_partial_bytes(M, r, K);            // U = X A^T
  size_t t = skinny_partial_bytes(M, r, N);               // dU = s dY B
  if (t > part) part = t;
  t = skinny_partial_bytes(N, r, M);                      // dB = s dY^T U
  if (t > part) part = t;
  t = skinny_partial_bytes(r, K, M);                      // dA = dU^T X
  if (t > part) part = t;
  p.total = p.part_off + align_up(part);
  return p;
}

bool nf4_ok(const nf4_tensor_t* w) {
  return w && w->codes && w->q8 && w->step;
}

int32_t nf4_supported(const nf4_tensor_t* w) {
  return (w->blocksize == QLORA_NF4_BLOCKSIZE && w->dq_blocksize == QLORA_NF4_DQ_BLOCKSIZE)
             ? QLORA_OK
             : QLORA_ERR_UNSUPPORTED;
}

inline int32_t launch_status(hipError_t e) { return e == hipSuccess ? QLORA_OK : QLORA_ERR_LAUNCH; }

// U = X A^T (unscaled), into ws_u [M][rp] (zero-padded) and optionally U_out [M][r].
hipError_t run_lora_down(const uint16_t* X, int64_t M, int64_t K, const uint16_t* A, int32_t r,
                         uint16_t* ws_u, uint16_t* U_out, float* part, hipStream_t stream) {
  SkinnyOp op{X, K, 1, A, K, 1, M, r, K};
  const int sp = skinny_splits(M, r, K);
  hipError_t e = launch_skinny_partial(op, sp, part, stream);
  if (e != hipSuccess) return e;
  return launch_skinny_finish(part, sp, M, r, 1.0f, ws_u, rank_pad(r), rank_pad(r), U_out, r,
                              stream);
}

}  // namespace

extern "C" {

const char* qlora_status_str(int32_t status) {
  switch (status) {
    case QLORA_OK: return "ok";
    case QLORA_ERR_INVALID: return "invalid argument (null pointer, size or alignment)";
    case QLORA_ERR_UNSUPPORTED: return "unsupported configuration (block sizes must be 64 and 256)";
    case QLORA_ERR_WORKSPACE: return "workspace too small";
    case QLORA_ERR_LAUNCH: return "HIP launch error";
    default: return "unknown status";
  }
}

void nf4_code_table(float* levels16, float* thresholds15) {
  if (levels16)
    for (int i = 0; i < 16; ++i) levels16[i] = level_f32(i);
  if (thresholds15)
    for (int i = 0; i < 15; ++i) thresholds15[i] = __builtin_bit_cast(float, kThr.bits[i]);
}

size_t nf4_storage_bytes(int64_t N, int64_t K) {
  if (N < 1 || K < 64 || (K % 64) != 0) return 0;
  const int64_t nb = N * K / 64;
  return (size_t)(N * K / 2) + (size_t)nb + 4 * (size_t)((nb + 255) / 256);
}

int32_t nf4_quantize(const float* W, int64_t N, int64_t K, int32_t blocksize,
                     int32_t dq_blocksize, uint8_t* codes, uint8_t* q8, float* step,
                     hipStream_t stream) {
  if (!W || !codes || !q8 || !step) return QLORA_ERR_INVALID;
  if (N < 1 || K < 64 || (K % 64) != 0 || N > ((int64_t)1 << 40) / K) return QLORA_ERR_INVALID;
  if (blocksize != QLORA_NF4_BLOCKSIZE || dq_blocksize != QLORA_NF4_DQ_BLOCKSIZE)
    return QLORA_ERR_UNSUPPORTED;
  if (!aligned16(W) || !aligned16(codes) || !aligned16(q8) || !aligned16(step))
    return QLORA_ERR_INVALID;
  return launch_status(launch_nf4_quantize(W, N * K / 64, codes, q8, step, stream));
}

int32_t nf4_dequantize(const nf4_tensor_t* w, uint16_t* W_bf16, hipStream_t stream) {
  if (!nf4_ok(w) || !W_bf16) return QLORA_ERR_INVALID;
  if (w->N < 1 || w->K < 64 || (w->K % 64) != 0) return QLORA_ERR_INVALID;
  const int32_t sup = nf4_supported(w);
  if (sup != QLORA_OK) return sup;
  if (!aligned16(w->codes) || !aligned16(w->q8) || !aligned16(w->step) || !aligned16(W_bf16))
    return QLORA_ERR_INVALID;
  return launch_status(launch_nf4_dequantize(w->codes, w->q8, w->step, w->N * w->K, W_bf16, stream));
}

size_t qlora_workspace_size(int64_t M, int64_t N, int64_t K, int32_t r, int32_t for_bwd) {
  if (!sizes_ok(M, N, K, r)) return 0;
  return for_bwd ? plan_bwd(M, N, K, r).total : plan_fwd(M, N, K, r).total;
}

}  // extern "C"

namespace {

inline hipError_t record(hipEvent_t ev, hipStream_t stream) {
  return ev ? hipEventRecord(ev, stream) : hipSuccess;
}

int32_t linear_fwd(const nf4_tensor_t* w, const uint16_t* X, int64_t M, const uint16_t* A,
                   const uint16_t* B, int32_t r, float s, uint16_t* Y, uint16_t* U_out, void* ws,
                   size_t ws_bytes, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  if (!nf4_ok(w) || !X || !A || !B || !Y || !ws) return QLORA_ERR_INVALID;
  const int32_t sup = nf4_supported(w);
  if (sup != QLORA_OK) return sup;
  const int64_t N = w->N, K = w->K;
  if (!sizes_ok(M, N, K, r) || !isfinite(s)) return QLORA_ERR_INVALID;
  if (!aligned16(w->codes) || !aligned16(w->q8) || !aligned16(w->step) || !aligned16(X) ||
      !aligned16(A) || !aligned16(B) || !aligned16(Y) || !aligned16(ws) ||
      (U_out && !aligned16(U_out)))
    return QLORA_ERR_INVALID;
  const FwdPlan pl = plan_fwd(M, N, K, r);
  if (ws_bytes < pl.total) return QLORA_ERR_WORKSPACE;

  char* base = static_cast<char*>(ws);
  uint16_t* ws_u = reinterpret_cast<uint16_t*>(base + pl.u_off);
  float* part = reinterpret_cast<float*>(base + pl.part_off);
  const Nf4View v{w->codes, w->q8, w->step, N, K};

  hipError_t e = run_lora_down(X, M, K, A, r, ws_u, U_out, part, stream);
  if (e != hipSuccess) return QLORA_ERR_LAUNCH;
  if (record(ev0, stream) != hipSuccess) return QLORA_ERR_LAUNCH;
  if (M <= kGemvMaxM) {
    e = launch_qgemv_partial(v, X, M, pl.gemv_splits_n, part, stream);
    if (e != hipSuccess || record(ev1, stream) != hipSuccess) return QLORA_ERR_LAUNCH;
    e = launch_gemv_finish(part, pl.gemv_splits_n, M, N, ws_u, rank_pad(r), B, r, s, Y, stream);
  } else {
    e = launch_qgemm_fwd(v, X, M, ws_u, rank_pad(r), B, r, s, Y, stream);
    if (e == hipSuccess) e = record(ev1, stream);
  }
  return launch_status(e);
}

int32_t linear_bwd(const nf4_tensor_t* w, const uint16_t* X, const uint16_t* dY, int64_t M,
                   const uint16_t* A, const uint16_t* B, const uint16_t* U, int32_t r, float s,
                   uint16_t* dX, uint16_t* dA, uint16_t* dB, void* ws, size_t ws_bytes,
                   hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  if (!nf4_ok(w) || !X || !dY || !A || !B || !dA || !dB || !ws) return QLORA_ERR_INVALID;
  const int32_t sup = nf4_supported(w);
  if (sup != QLORA_OK) return sup;
  const int64_t N = w->N, K = w->K;
  if (!sizes_ok(M, N, K, r) || !isfinite(s)) return QLORA_ERR_INVALID;
  if (!aligned16(w->codes) || !aligned16(w->q8) || !aligned16(w->step) || !aligned16(X) ||
      !aligned16(dY) || !aligned16(A) || !aligned16(B) || !aligned16(dA) || !aligned16(dB) ||
      !aligned16(ws) || (U && !aligned16(U)) || (dX && !aligned16(dX)))
    return QLORA_ERR_INVALID;
  const BwdPlan pl = plan_bwd(M, N, K, r);
  if (ws_bytes < pl.total) return QLORA_ERR_WORKSPACE;

  char* base = static_cast<char*>(ws);
  uint16_t* ws_u = reinterpret_cast<uint16_t*>(base + pl.u_off);
  uint16_t* ws_du = reinterpret_cast<uint16_t*>(base + pl.du_off);
  float* part = reinterpret_cast<float*>(base + pl.part_off);
  const int64_t rp = rank_pad(r);
  hipError_t e;

  // U = X A^T unless the caller kept it from the forward pass.
  const uint16_t* Uuse = U;
  int64_t ldu = r;
  if (!Uuse) {
    e = run_lora_down(X, M, K, A, r, ws_u, nullptr, part, stream);
    if (e != hipSuccess) return QLORA_ERR_LAUNCH;
    Uuse = ws_u;
    ldu = rp;
  }

  // dU = s dY B  -> ws_du [M][rp]
  {
    SkinnyOp op{dY, N, 1, B, 1, r, M, r, N};
    const int sp = skinny_splits(M, r, N);
    if ((e = launch_skinny_partial(op, sp, part, stream)) != hipSuccess) return QLORA_ERR_LAUNCH;
    if ((e = launch_skinny_finish(part, sp, M, r, s, ws_du, rp, rp, nullptr, 0, stream)) != hipSuccess)
      return QLORA_ERR_LAUNCH;
  }
  // dB = s dY^T U -> dB [N][r]
  {
    SkinnyOp op{dY, 1, N, Uuse, 1, ldu, N, r, M};
    const int sp = skinny_splits(N, r, M);
    if ((e = launch_skinny_partial(op, sp, part, stream)) != hipSuccess) return QLORA_ERR_LAUNCH;
    if ((e = launch_skinny_finish(part, sp, N, r, s, dB, r, r, nullptr, 0, stream)) != hipSuccess)
      return QLORA_ERR_LAUNCH;
  }
  // dA = dU^T X -> dA [r][K]
  {
    SkinnyOp op{ws_du, 1, rp, X, 1, K, r, K, M};
    const int sp = skinny_splits(r, K, M);
    if ((e = launch_skinny_partial(op, sp, part, stream)) != hipSuccess) return QLORA_ERR_LAUNCH;
    if ((e = launch_skinny_finish(part, sp, r, K, 1.0f, dA, K, K, nullptr, 0, stream)) != hipSuccess)
      return QLORA_ERR_LAUNCH;
  }
  // dX = dY W + dU A
  if (dX) {
    const Nf4View v{w->codes, w->q8, w->step, N, K};
    if (record(ev0, stream) != hipSuccess) return QLORA_ERR_LAUNCH;
    e = launch_qgemm_bwd(v, dY, M, ws_du, rp, A, r, dX, stream);
    if (e != hipSuccess || record(ev1, stream) != hipSuccess) return QLORA_ERR_LAUNCH;
  }
  return QLORA_OK;
}

}  // namespace

extern "C" {

int32_t qlora_linear_fwd(const nf4_tensor_t* w, const uint16_t* X, int64_t M, const uint16_t* A,
                         const uint16_t* B, int32_t r, float s, uint16_t* Y, uint16_t* U_out,
                         void* ws, size_t ws_bytes, hipStream_t stream) {
  return linear_fwd(w, X, M, A, B, r, s, Y, U_out, ws, ws_bytes, stream, nullptr, nullptr);
}

int32_t qlora_linear_fwd_ev(const nf4_tensor_t* w, const uint16_t* X, int64_t M,
                            const uint16_t* A, const uint16_t* B, int32_t r, float s, uint16_t* Y,
                            uint16_t* U_out, void* ws, size_t ws_bytes, hipStream_t stream,
                            hipEvent_t ev_begin, hipEvent_t ev_end) {
  return linear_fwd(w, X, M, A, B, r, s, Y, U_out, ws, ws_bytes, stream, ev_begin, ev_end);
}

int32_t qlora_linear_bwd(const nf4_tensor_t* w, const uint16_t* X, const uint16_t* dY, int64_t M,
                         const uint16_t* A, const uint16_t* B, const uint16_t* U, int32_t r,
                         float s, uint16_t* dX, uint16_t* dA, uint16_t* dB, void* ws,
                         size_t ws_bytes, hipStream_t stream) {
  return linear_bwd(w, X, dY, M, A, B, U, r, s, dX, dA, dB, ws, ws_bytes, stream, nullptr,
                    nullptr);
}

int32_t qlora_linear_bwd_ev(const nf4_tensor_t* w, const uint16_t* X, const uint16_t* dY,
                            int64_t M, const uint16_t* A, const uint16_t* B, const uint16_t* U,
                            int32_t r, float s, uint16_t* dX, uint16_t* dA, uint16_t* dB,
                            void* ws, size_t ws_bytes, hipStream_t stream, hipEvent_t ev_begin,
                            hipEvent_t ev_end) {
  return linear_bwd(w, X, dY, M, A, B, U, r, s, dX, dA, dB, ws, ws_bytes, stream, ev_begin,
                    ev_end);
}

}  // extern "C"
