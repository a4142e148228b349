// C ABI of the NF4 + LoRA linear layer: argument checks, workspace carving
// and the launch sequence of each call.  The declarations, with the meaning,
// layout and ownership of every argument, are in include/qlora_nf4.h.
#include "../../include/qlora_nf4.h"

#include <math.h>

#include <algorithm>
#include <mutex>

#include "kernels.hpp"

using namespace qn;

namespace {

inline int32_t launch_status(hipError_t e) { return e == hipSuccess ? QLORA_OK : QLORA_ERR_LAUNCH; }

constexpr size_t kAlign = 256;

inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
inline int64_t rank_pad(int32_t r) { return ((int64_t)r + 63) / 64 * 64; }

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct FwdPlan {
  size_t u_off, part_off, total;
};

// Backward: with U given, [dU | dB] then [dA]; otherwise [U | dU] then
// [dB | dA].  Slot 0 and slot 1 of a launch pair have their own partial
// buffer; the second pair reuses them.
struct BwdPlan {
  size_t u_off, du_off, part0_off, part1_off, total;
};

bool sizes_ok(int64_t M, int64_t N, int64_t K, int32_t r) {
  return M >= 1 && N >= 1 && K >= 64 && (K % 64) == 0 && (N % 8) == 0 && r >= 1 &&
         r <= QLORA_MAX_RANK && M <= ((int64_t)1 << 31) && N <= QLORA_LINEAR_MAX_NK &&
         K <= QLORA_LINEAR_MAX_NK;
}

FwdPlan plan_fwd(int64_t M, int64_t N, int64_t K, int32_t r) {
  FwdPlan p{};
  const int64_t rp = rank_pad(r);
  p.u_off = 0;
  p.part_off = align_up((size_t)M * rp * 2);
  (void)N;
  const size_t part = gemv_fits(M, r, K) ? gemv_workspace_bytes(M, r, K) : skinny_partial_bytes(M, r, K);
  p.total = p.part_off + align_up(part);
  return p;
}

BwdPlan plan_bwd(int64_t M, int64_t N, int64_t K, int32_t r) {
  BwdPlan p{};
  const int64_t rp = rank_pad(r);
  p.u_off = 0;
  p.du_off = align_up((size_t)M * rp * 2);
  // slot 0: U or dU, then dB;  slot 1: dU or dB, then dA
  const size_t b_u = skinny_partial_bytes(M, r, K), b_du = skinny_partial_bytes(M, r, N),
               b_db = skinny_partial_bytes(N, r, M), b_da = skinny_partial_bytes(r, K, M);
  const size_t part0 = std::max(std::max(b_u, b_du), b_db);
  const size_t part1 = std::max(std::max(b_du, b_db), b_da);
  p.part0_off = p.du_off + align_up((size_t)M * rp * 2);
  p.part1_off = p.part0_off + align_up(part0);
  p.total = p.part1_off + align_up(part1);
  return p;
}

bool nf4_ok(const nf4_tensor_t* w) {
  return w && w->codes && w->q8 && w->step;
}

inline bool code_ok(int32_t code_type) {
  return code_type == QLORA_CODE_NF4 || code_type == QLORA_CODE_FP4 ||
         code_type == QLORA_CODE_NF3 || code_type == QLORA_CODE_NF2;
}

inline bool user_type(int32_t code_type) {
  return code_type == QLORA_CODE_USER4 || code_type == QLORA_CODE_USER3 ||
         code_type == QLORA_CODE_USER2;
}

// Built-in or caller-codebook code type.
inline bool any_code_ok(int32_t code_type) { return code_ok(code_type) || user_type(code_type); }

inline int code_bits(int32_t code_type) {
  return with_any_code(code_type, [](auto ct) { return decltype(ct)::kBits; });
}

// The table of a caller's codebook (user_type(code_type)): the values must
// be finite, |v| <= 1, and 0 or |v| >= 2^-20, so that the sum of any two is
// exact in fp64 and each threshold is its exact midpoint rounded down.  The
// rest is the built-in tables' construction over the first 2^k codes.
// Returns the number of thresholds, or -1 if the values break the contract.
int user_table(int32_t code_type, const float* levels, UserTable* out) {
  if (!levels) return -1;
  const int n = 1 << code_bits(code_type);
  uint32_t lv[16] = {};
  for (int c = 0; c < n; ++c) {
    const float v = levels[c];
    if (!isfinite(v) || fabsf(v) > 1.0f || (v != 0.0f && fabsf(v) < QLORA_USER_MIN_MAGNITUDE))
      return -1;
    lv[c] = __builtin_bit_cast(uint32_t, v);
  }
  const CodeTable t = make_code_table(lv, n);
  if (!code_table_sound(t)) return -1;  // not reached under the contract
  UserTable u{};
  for (int c = 0; c < 16; ++c) u.level[c] = __builtin_bit_cast(float, t.level[c]);
  for (int i = 0; i < 15; ++i)
    u.thr[i] = i + 1 < t.ndist ? __builtin_bit_cast(float, t.thr[i]) : __builtin_inff();
  uint64_t map = 0;
  for (int k = 0; k < t.ndist; ++k) map |= (uint64_t)t.dist_code[k] << (4 * k);
  u.code_lo = (uint32_t)map;
  u.code_hi = (uint32_t)(map >> 32);
  if (out) *out = u;
  return t.ndist - 1;
}

// The layer kernels address the packed codes with 32-bit buffer offsets.
bool state_fits(const nf4_tensor_t* w) {
  const int64_t bits = code_bits(w->code_type);
  return w->N * w->K / 8 * bits < ((int64_t)1 << 31);
}

// Block sizes 64, 128, 256 as 64 << shift; -1 for others.
inline int bshift_of(int32_t blocksize) {
  return blocksize == 64 ? 0 : blocksize == 128 ? 1 : blocksize == 256 ? 2 : -1;
}

// Configuration of a quantized weight: a supported block size, DQ block
// size and code type (else QLORA_ERR_UNSUPPORTED), K a multiple of the
// block size and, for a caller's codebook, values within the contract (else
// QLORA_ERR_INVALID).
int32_t nf4_supported(const nf4_tensor_t* w) {
  if (bshift_of(w->blocksize) < 0 || w->dq_blocksize != QLORA_NF4_DQ_BLOCKSIZE ||
      !any_code_ok(w->code_type))
    return QLORA_ERR_UNSUPPORTED;
  if (user_type(w->code_type) && user_table(w->code_type, w->levels, nullptr) < 0)
    return QLORA_ERR_INVALID;
  return (w->K % w->blocksize) == 0 ? QLORA_OK : QLORA_ERR_INVALID;
}

// For a tensor nf4_supported accepted.
inline Nf4View view_of(const nf4_tensor_t* w) {
  Nf4View v{w->codes, w->q8, w->step, w->N, w->K, w->code_type, bshift_of(w->blocksize), {}};
  if (user_type(w->code_type)) user_table(w->code_type, w->levels, &v.ut);
  return v;
}

size_t config_bytes(int32_t code_type, int32_t blocksize, int64_t N, int64_t K) {
  if (!any_code_ok(code_type) || bshift_of(blocksize) < 0 || N < 1 || K < 64 || (K % 64) != 0 ||
      (K % blocksize) != 0)
    return 0;
  const int64_t nb = N * K / blocksize;
  const int64_t bits = code_bits(code_type);
  return (size_t)(N * K / 8 * bits) + (size_t)nb + 4 * (size_t)((nb + 255) / 256);
}

static_assert(CodeNF4::kId == QLORA_CODE_NF4 && CodeFP4::kId == QLORA_CODE_FP4 &&
                  CodeNF3::kId == QLORA_CODE_NF3 && CodeNF2::kId == QLORA_CODE_NF2,
              "code type ids of the ABI and of the kernels agree");

template <class CT>
int32_t copy_table(float* levels16, float* thresholds15) {
  if (levels16)
    for (int i = 0; i < 16; ++i) levels16[i] = code_value<CT>(i);
  if (thresholds15)
    for (int i = 0; i < 15; ++i)
      thresholds15[i] = i + 1 < CT::table.ndist ? __builtin_bit_cast(float, CT::table.thr[i]) : 0.0f;
  return CT::table.ndist - 1;
}

// levels: the caller's codebook for a user code type, else null.
int32_t quantize(const float* W, int64_t N, int64_t K, int32_t code_type, const float* levels,
                 int32_t blocksize, int32_t dq_blocksize, uint8_t* codes, uint8_t* q8,
                 float* step, hipStream_t stream) {
  if (!W || !codes || !q8 || !step) return QLORA_ERR_INVALID;
  if (N < 1 || K < 64 || (K % 64) != 0 || N > ((int64_t)1 << 40) / K) return QLORA_ERR_INVALID;
  const int bs = bshift_of(blocksize);
  if (bs < 0 || dq_blocksize != QLORA_NF4_DQ_BLOCKSIZE || !any_code_ok(code_type))
    return QLORA_ERR_UNSUPPORTED;
  if ((K % blocksize) != 0) return QLORA_ERR_INVALID;
  UserTable ut{};
  if (user_type(code_type) && user_table(code_type, levels, &ut) < 0) return QLORA_ERR_INVALID;
  if (!aligned16(W) || !aligned16(codes) || !aligned16(q8) || !aligned16(step))
    return QLORA_ERR_INVALID;
  return launch_status(
      launch_nf4_quantize(W, N * K / blocksize, codes, q8, step, code_type, bs, &ut, stream));
}

}  // namespace

extern "C" {

const char* qlora_status_str(int32_t status) {
  switch (status) {
    case QLORA_OK: return "ok";
    case QLORA_ERR_INVALID: return "invalid argument (null pointer, size or alignment)";
    case QLORA_ERR_UNSUPPORTED:
      return "unsupported configuration (block size, double-quantization block size or code type)";
    case QLORA_ERR_WORKSPACE: return "workspace too small";
    case QLORA_ERR_LAUNCH: return "HIP launch error";
    case QLORA_ERR_INFEASIBLE: return "no choice fits the budget";
    default: return "unknown status";
  }
}

void nf4_code_table(float* levels16, float* thresholds15) {
  copy_table<CodeNF4>(levels16, thresholds15);
}

int32_t qlora_code_table(int32_t code_type, float* levels16, float* thresholds15) {
  if (!code_ok(code_type)) return QLORA_ERR_UNSUPPORTED;
  return with_code(code_type, [&](auto ct) {
    return copy_table<decltype(ct)>(levels16, thresholds15);
  });
}

size_t qlora_storage_bytes(int32_t code_type, int64_t N, int64_t K) {
  return config_bytes(code_type, QLORA_NF4_BLOCKSIZE, N, K);
}

size_t qlora_config_bytes(int32_t code_type, int32_t blocksize, int64_t N, int64_t K) {
  return config_bytes(code_type, blocksize, N, K);
}

size_t nf4_storage_bytes(int64_t N, int64_t K) {
  if (N < 1 || K < 64 || (K % 64) != 0) return 0;
  const int64_t nb = N * K / 64;
  return (size_t)(N * K / 2) + (size_t)nb + 4 * (size_t)((nb + 255) / 256);
}

int32_t nf4_quantize(const float* W, int64_t N, int64_t K, int32_t blocksize,
                     int32_t dq_blocksize, uint8_t* codes, uint8_t* q8, float* step,
                     hipStream_t stream) {
  return quantize(W, N, K, QLORA_CODE_NF4, nullptr, blocksize, dq_blocksize, codes, q8, step,
                  stream);
}

int32_t qlora_quantize(const float* W, int64_t N, int64_t K, int32_t code_type,
                       int32_t blocksize, int32_t dq_blocksize, uint8_t* codes, uint8_t* q8,
                       float* step, hipStream_t stream) {
  return quantize(W, N, K, code_type, nullptr, blocksize, dq_blocksize, codes, q8, step, stream);
}

int32_t qlora_quantize_user(const float* W, int64_t N, int64_t K, int32_t code_type,
                            const float* levels, int32_t blocksize, int32_t dq_blocksize,
                            uint8_t* codes, uint8_t* q8, float* step, hipStream_t stream) {
  if (!user_type(code_type)) return QLORA_ERR_UNSUPPORTED;
  return quantize(W, N, K, code_type, levels, blocksize, dq_blocksize, codes, q8, step, stream);
}

int32_t qlora_user_table(int32_t code_type, const float* levels, float* thresholds15) {
  if (!user_type(code_type)) return QLORA_ERR_UNSUPPORTED;
  UserTable u;
  const int n = user_table(code_type, levels, &u);
  if (n < 0) return QLORA_ERR_INVALID;
  if (thresholds15)
    for (int i = 0; i < 15; ++i) thresholds15[i] = i < n ? u.thr[i] : 0.0f;
  return n;
}

int32_t nf4_dequantize(const nf4_tensor_t* w, uint16_t* W_bf16, hipStream_t stream) {
  if (!nf4_ok(w) || !W_bf16) return QLORA_ERR_INVALID;
  if (w->N < 1 || w->K < 64 || (w->K % 64) != 0) return QLORA_ERR_INVALID;
  const int32_t sup = nf4_supported(w);
  if (sup != QLORA_OK) return sup;
  if (!aligned16(w->codes) || !aligned16(w->q8) || !aligned16(w->step) || !aligned16(W_bf16))
    return QLORA_ERR_INVALID;
  const Nf4View v = view_of(w);
  return launch_status(launch_nf4_dequantize(w->codes, w->q8, w->step, w->N * w->K, W_bf16,
                                             w->code_type, v.bshift, &v.ut, stream));
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

// Every check of the forward call's arguments except the workspace.
int32_t check_fwd(const nf4_tensor_t* w, const uint16_t* X, int64_t M, const uint16_t* A,
                  const uint16_t* B, int32_t r, float s, const uint16_t* Y,
                  const uint16_t* U_out) {
  if (!nf4_ok(w) || !X || !A || !B || !Y) return QLORA_ERR_INVALID;
  const int32_t sup = nf4_supported(w);
  if (sup != QLORA_OK) return sup;
  if (!sizes_ok(M, w->N, w->K, r) || !isfinite(s) || !state_fits(w)) return QLORA_ERR_INVALID;
  if (!aligned16(w->codes) || !aligned16(w->q8) || !aligned16(w->step) || !aligned16(X) ||
      !aligned16(A) || !aligned16(B) || !aligned16(Y) || (U_out && !aligned16(U_out)))
    return QLORA_ERR_INVALID;
  return QLORA_OK;
}

int32_t linear_fwd(const nf4_tensor_t* w, const uint16_t* X, int64_t M, const uint16_t* A,
                   const uint16_t* B, int32_t r, float s, uint16_t* Y, uint16_t* U_out, void* ws,
                   size_t ws_bytes, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  const int32_t chk = check_fwd(w, X, M, A, B, r, s, Y, U_out);
  if (chk != QLORA_OK) return chk;
  if (!ws || !aligned16(ws)) return QLORA_ERR_INVALID;
  const int64_t N = w->N, K = w->K;
  const FwdPlan pl = plan_fwd(M, N, K, r);
  if (ws_bytes < pl.total) return QLORA_ERR_WORKSPACE;

  char* base = static_cast<char*>(ws);
  uint16_t* ws_u = reinterpret_cast<uint16_t*>(base + pl.u_off);
  float* part = reinterpret_cast<float*>(base + pl.part_off);
  const Nf4View v = view_of(w);
  const int64_t rp = rank_pad(r);

  if (gemv_fits(M, r, K))
    return launch_status(launch_qgemv(v, X, M, A, B, r, s, Y, U_out, part, stream, ev0, ev1));

  // U = X A^T into ws_u [M][rp] (zero-padded) and U_out [M][r].
  const SkinnyJob ju = make_job(SkinnyOp{X, K, 1, A, K, 1, M, r, K}, 1.0f, ws_u, rp, rp, U_out, r,
                                part);
  hipError_t e = launch_skinny(&ju, 1, stream);
  if (e != hipSuccess) return QLORA_ERR_LAUNCH;
  if (record(ev0, stream) != hipSuccess) return QLORA_ERR_LAUNCH;
  e = launch_qgemm_fwd(v, X, M, ws_u, rp, B, r, s, Y, stream);
  if (e == hipSuccess) e = record(ev1, stream);
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
  if (!sizes_ok(M, N, K, r) || !isfinite(s) || !state_fits(w)) return QLORA_ERR_INVALID;
  if (!aligned16(w->codes) || !aligned16(w->q8) || !aligned16(w->step) || !aligned16(X) ||
      !aligned16(dY) || !aligned16(A) || !aligned16(B) || !aligned16(dA) || !aligned16(dB) ||
      !aligned16(ws) || (U && !aligned16(U)) || (dX && !aligned16(dX)))
    return QLORA_ERR_INVALID;
  const BwdPlan pl = plan_bwd(M, N, K, r);
  if (ws_bytes < pl.total) return QLORA_ERR_WORKSPACE;

  char* base = static_cast<char*>(ws);
  uint16_t* ws_u = reinterpret_cast<uint16_t*>(base + pl.u_off);
  uint16_t* ws_du = reinterpret_cast<uint16_t*>(base + pl.du_off);
  float* part0 = reinterpret_cast<float*>(base + pl.part0_off);
  float* part1 = reinterpret_cast<float*>(base + pl.part1_off);
  const int64_t rp = rank_pad(r);
  hipError_t e;

  // dU = s dY B -> ws_du [M][rp] (zero-padded)
  const SkinnyOp op_du{dY, N, 1, B, 1, r, M, r, N};
  // dA = dU^T X -> dA [r][K]
  const SkinnyOp op_da{ws_du, 1, rp, X, 1, K, r, K, M};
  if (U) {
    // dB = s dY^T U -> dB [N][r], with the caller's U [M][r]
    const SkinnyJob j1[2] = {
        make_job(op_du, s, ws_du, rp, rp, nullptr, 0, part0),
        make_job(SkinnyOp{dY, 1, N, U, 1, r, N, r, M}, s, dB, r, r, nullptr, 0, part1)};
    if ((e = launch_skinny(j1, 2, stream)) != hipSuccess) return QLORA_ERR_LAUNCH;
    const SkinnyJob j2 = make_job(op_da, 1.0f, dA, K, K, nullptr, 0, part1);
    if ((e = launch_skinny(&j2, 1, stream)) != hipSuccess) return QLORA_ERR_LAUNCH;
  } else {
    // U = X A^T -> ws_u, then dB with ws_u
    const SkinnyJob j1[2] = {
        make_job(SkinnyOp{X, K, 1, A, K, 1, M, r, K}, 1.0f, ws_u, rp, rp, nullptr, 0, part0),
        make_job(op_du, s, ws_du, rp, rp, nullptr, 0, part1)};
    if ((e = launch_skinny(j1, 2, stream)) != hipSuccess) return QLORA_ERR_LAUNCH;
    const SkinnyJob j2[2] = {
        make_job(SkinnyOp{dY, 1, N, ws_u, 1, rp, N, r, M}, s, dB, r, r, nullptr, 0, part0),
        make_job(op_da, 1.0f, dA, K, K, nullptr, 0, part1)};
    if ((e = launch_skinny(j2, 2, stream)) != hipSuccess) return QLORA_ERR_LAUNCH;
  }

  // dX = dY W + dU A
  if (dX) {
    const Nf4View v = view_of(w);
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

// ---------------------------------------------------------------------------
// Forward pass without a caller workspace: the scratch is this file's fixed
// device array.  Host code never passes the array's name to a kernel (on the
// host it is only a stand-in for the symbol); it passes the device address
// that hipGetSymbolAddress returns, fetched once per device with that device
// current and cached per device.
// ---------------------------------------------------------------------------
namespace {

__device__ __align__(256) unsigned char scratch[QLORA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int32_t scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return QLORA_ERR_LAUNCH;
  if (dev < 0 || dev >= kMaxDevices) return QLORA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return QLORA_ERR_LAUNCH;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return QLORA_OK;
}

}  // namespace

extern "C" int32_t qlora_linear_fwd_noalloc(const nf4_tensor_t* w, const uint16_t* X, int64_t M,
                                            const uint16_t* A, const uint16_t* B, int32_t r,
                                            float s, uint16_t* Y, uint16_t* U_out,
                                            hipStream_t stream) {
  // Argument errors first, as qlora_linear_fwd reports them, so that nothing
  // else (not even the symbol lookup) happens for a rejected call.
  const int32_t chk = check_fwd(w, X, M, A, B, r, s, Y, U_out);
  if (chk != QLORA_OK) return chk;
  if (plan_fwd(M, w->N, w->K, r).total > QLORA_NOALLOC_SCRATCH_BYTES) return QLORA_ERR_WORKSPACE;
  void* ws = nullptr;
  const int32_t st = scratch_address(&ws);
  if (st != QLORA_OK) return st;
  return linear_fwd(w, X, M, A, B, r, s, Y, U_out, ws, QLORA_NOALLOC_SCRATCH_BYTES, stream,
                    nullptr, nullptr);
}

extern "C" int32_t qlora_stream_read(const void* src, size_t bytes, uint32_t* sink,
                                     hipStream_t stream) {
  if (!src || !sink || bytes == 0 || (bytes % 16) != 0 || !aligned16(src) ||
      ((uintptr_t)sink & 3u) != 0)
    return QLORA_ERR_INVALID;
  return launch_status(qn::launch_stream_read(src, bytes, sink, QLORA_STREAM_GRID, stream));
}

extern "C" {

size_t qlora_lq_workspace_size(int64_t N, int64_t K, int32_t r, int32_t l) {
  if (N < 1 || K < 64 || (K % 64) != 0 || r < 1 || l <= r || l > QLORA_LQ_MAX_L || (l % 16) != 0 ||
      N > ((int64_t)1 << 40) / K)
    return 0;
  return qn::lq_workspace_bytes(N, K, l);
}

int32_t qlora_lq_init(const float* W, int64_t N, int64_t K, int32_t code_type, int32_t r,
                      int32_t l, const float* omega, int32_t iters, int32_t power_iters,
                      int32_t start, float s, uint8_t* codes, uint8_t* q8, float* step,
                      uint16_t* A, uint16_t* B, float* L1, float* L2t, void* ws, size_t ws_bytes,
                      hipStream_t stream) {
  if (!W || !omega || !codes || !q8 || !step || !A || !B || !L1 || !L2t || !ws)
    return QLORA_ERR_INVALID;
  const size_t need = qlora_lq_workspace_size(N, K, r, l);
  if (need == 0 || iters < 1 || iters > 64 || power_iters < 0 || power_iters > 16 ||
      (start != QLORA_LQ_START_SVD && start != QLORA_LQ_START_QUANTIZE) || !isfinite(s) ||
      s == 0.0f)
    return QLORA_ERR_INVALID;
  if (!code_ok(code_type)) return QLORA_ERR_UNSUPPORTED;
  if (!aligned16(W) || !aligned16(omega) || !aligned16(codes) || !aligned16(q8) ||
      !aligned16(step) || !aligned16(A) || !aligned16(B) || !aligned16(L1) || !aligned16(L2t) ||
      ((uintptr_t)ws & 255u) != 0)
    return QLORA_ERR_INVALID;
  if (ws_bytes < need) return QLORA_ERR_WORKSPACE;
  const qn::LqArgs a{W, N, K, code_type, r, l, omega, iters, power_iters, start, s,
                     codes, q8, step, A, B, L1, L2t, ws};
  return launch_status(qn::launch_lq_init(a, stream));
}

}  // extern "C"

extern "C" {

size_t qlora_config_error_workspace_size(int64_t N, int64_t K, int32_t code_type,
                                         int32_t blocksize, int32_t with_lowrank) {
  if (!code_ok(code_type) || bshift_of(blocksize) < 0 || N < 1 || K < 64 || (K % 64) != 0 ||
      (K % blocksize) != 0 || N > ((int64_t)1 << 40) / K)
    return 0;
  const int bits = with_code(code_type, [](auto ct) { return decltype(ct)::kBits; });
  return qn::quant_error_workspace_bytes(N, K, bits, bshift_of(blocksize), with_lowrank != 0);
}

size_t qlora_quant_error_workspace_size(int64_t N, int64_t K, int32_t code_type,
                                        int32_t with_lowrank) {
  return qlora_config_error_workspace_size(N, K, code_type, QLORA_NF4_BLOCKSIZE, with_lowrank);
}

int32_t qlora_config_error(const float* W, int64_t N, int64_t K, int32_t code_type,
                           int32_t blocksize, const float* L1, const float* L2t, int32_t r,
                           double* sq_err, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!W || !sq_err || !ws || ((L1 == nullptr) != (L2t == nullptr))) return QLORA_ERR_INVALID;
  if (!code_ok(code_type) || bshift_of(blocksize) < 0) return QLORA_ERR_UNSUPPORTED;
  const size_t need =
      qlora_config_error_workspace_size(N, K, code_type, blocksize, L1 != nullptr);
  if (need == 0) return QLORA_ERR_INVALID;
  if (L1 && (r < 1 || r > QLORA_LQ_MAX_L || !aligned16(L1) || !aligned16(L2t)))
    return QLORA_ERR_INVALID;
  if (!aligned16(W) || ((uintptr_t)sq_err & 7u) != 0 || ((uintptr_t)ws & 255u) != 0)
    return QLORA_ERR_INVALID;
  if (ws_bytes < need) return QLORA_ERR_WORKSPACE;
  return launch_status(qn::launch_quant_error(W, N, K, code_type, bshift_of(blocksize), L1, L2t,
                                              r, sq_err, ws, stream));
}

int32_t qlora_quant_error(const float* W, int64_t N, int64_t K, int32_t code_type,
                          const float* L1, const float* L2t, int32_t r, double* sq_err, void* ws,
                          size_t ws_bytes, hipStream_t stream) {
  return qlora_config_error(W, N, K, code_type, QLORA_NF4_BLOCKSIZE, L1, L2t, r, sq_err, ws,
                            ws_bytes, stream);
}

int32_t qlora_ilp_plan(int32_t n_matrices, int32_t n_configs, const double* err,
                       const int64_t* bytes, int64_t budget, int32_t* choice, double* total_err,
                       int64_t* total_bytes) {
  if (n_matrices < 1 || n_configs < 1 || n_configs > 64 || n_matrices > (1 << 20) || !err ||
      !bytes || !choice || !total_err || !total_bytes || budget < 0)
    return QLORA_ERR_INVALID;
  for (int64_t i = 0; i < (int64_t)n_matrices * n_configs; ++i)
    if (!isfinite(err[i]) || bytes[i] < 0) return QLORA_ERR_INVALID;
  return qn::ilp_plan(n_matrices, n_configs, err, bytes, budget, choice, total_err, total_bytes)
             ? QLORA_OK
             : QLORA_ERR_INFEASIBLE;
}

}  // extern "C"
