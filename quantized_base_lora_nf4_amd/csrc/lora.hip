// Small-rank LoRA products: U = X A^T, dU = s dY B, dB = s dY^T U and
// dA = dU^T X.  LoRA trains only a low-rank pair beside the frozen weight
// ("QLoRA: fine-tuning a 65B model on one GPU", section "Where the memory
// goes"), so one side of each of these products is the rank r (<= 256) and
// the contraction is long (K, N or M): they are bound by reading X or dY.
//
// One generic MFMA kernel computes C[I, J] = scale * sum_c Aop(i, c) Bop(c, j)
// for up to two independent products in one launch.  Each product's output
// is cut into 64 x 64 tiles and its contraction into `splits` equal slices;
// a workgroup computes one (tile, slice) partial in fp32.  A product with one
// slice is finished in place; otherwise the partials go to the workspace and
// a second launch adds the slices in slice order, scales and rounds to bf16
// (for both products of the first launch at once).  No atomics and no
// cross-workgroup fences (a device-scope fence writes back and invalidates
// the per-XCD L2s), and the summation order is fixed, so results are
// bit-reproducible.
//
// Tiles are 64 x 64 outputs per 256-thread workgroup (2 x 2 waves of one
// 32 x 32 MFMA tile each), 64-deep contraction steps staged through LDS.
// Operands move as 16-byte chunks: kept whole along the contraction, or
// scattered element-wise when the chunk runs along the output dimension (the
// transpose).  Misaligned operands fall back to element loads.
#include "kernels.hpp"

namespace qn {

namespace {

constexpr int SLD = 72;
constexpr int kSkinnyStep = 64;

struct Prob {
  SkinnyOp op;
  int64_t c_split;   // contraction length per slice (multiple of 64)
  float scale;
  uint16_t* out;     // out[i * o_si + j]; zero for J <= j < Jw
  int64_t o_si, Jw;
  uint16_t* out2;    // optional copy without the padding
  int64_t o2_si;
  float* part;       // [tiles][splits][64 * 64]
  int splits, tiles_j, tiles;
  int wg_begin;      // first workgroup id of this product
  bool a_vec, b_vec;
};

struct Launch {
  Prob p[2];
  int nprob;
};

// Operand tile staging, split into a global-load half (into registers, so
// the next step's loads are in flight while the current step computes) and
// an LDS-store half.  The tile is 64 x 64: element (x, c) of the operand is
// at src[x * sx + c * sc] and lands in T[x][c] (c contiguous in LDS); rows
// x >= X or columns c >= cend read as zero.  One of sx, sc is 1.  With
// `vec`, each thread moves two 16-byte chunks of eight contiguous elements:
// along c they are stored whole, along x they are scattered element-wise (a
// transpose).  Otherwise each thread moves 16 single elements.
struct OpRegs {
  u32x4 v[2];  // vec: two chunks; otherwise 16 elements packed in pairs
};

__device__ __forceinline__ void load_op(OpRegs& R, const uint16_t* src, int64_t sx, int64_t sc,
                                        int64_t x0, int64_t X, int64_t c0, int64_t cend,
                                        bool vec, int tid) {
  const bool c_fast = (sc == 1);
  if (vec) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int e = tid + 256 * q;
      const int xi = c_fast ? (e >> 3) : ((e & 7) * 8);
      const int ci = c_fast ? ((e & 7) * 8) : (e >> 3);
      const int64_t gx = x0 + xi, gc = c0 + ci;
      R.v[q] = u32x4{0u, 0u, 0u, 0u};
      if (gx < X && gc < cend)
        R.v[q] = *reinterpret_cast<const u32x4*>(src + (c_fast ? gx * sx + gc : gc * sc + gx));
    }
    return;
  }
  for (int q = 0; q < 16; ++q) {
    const int e = tid + 256 * q;
    const int xi = c_fast ? (e >> 6) : (e & 63);
    const int ci = c_fast ? (e & 63) : (e >> 6);
    const int64_t gx = x0 + xi, gc = c0 + ci;
    const uint32_t v = (gx < X && gc < cend) ? src[gx * sx + gc * sc] : 0u;
    const uint32_t w = R.v[q >> 3][(q >> 1) & 3];
    R.v[q >> 3][(q >> 1) & 3] = (q & 1) ? ((w & 0xffffu) | (v << 16)) : v;
  }
}

__device__ __forceinline__ void store_op(uint16_t* T, const OpRegs& R, bool c_fast, bool vec,
                                         int tid) {
  if (vec) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int e = tid + 256 * q;
      if (c_fast) {
        *reinterpret_cast<u32x4*>(T + (e >> 3) * SLD + (e & 7) * 8) = R.v[q];
      } else {
        const int ci = e >> 3, xi = (e & 7) * 8;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          T[(xi + 2 * j) * SLD + ci] = (uint16_t)(R.v[q][j] & 0xffffu);
          T[(xi + 2 * j + 1) * SLD + ci] = (uint16_t)(R.v[q][j] >> 16);
        }
      }
    }
    return;
  }
  for (int q = 0; q < 16; ++q) {
    const int e = tid + 256 * q;
    const int xi = c_fast ? (e >> 6) : (e & 63);
    const int ci = c_fast ? (e & 63) : (e >> 6);
    const uint32_t w = R.v[q >> 3][(q >> 1) & 3];
    T[xi * SLD + ci] = (uint16_t)((q & 1) ? (w >> 16) : (w & 0xffffu));
  }
}

// Write one finished output element (and the optional unpadded copy).
__device__ __forceinline__ void put(const Prob& P, int64_t i, int64_t j, float v) {
  const uint16_t b = f32_to_bf16(v * P.scale);
  P.out[i * P.o_si + j] = b;
  if (P.out2) P.out2[i * P.o2_si + j] = b;
}

// kVec: every operand of every product in the launch moves as 16-byte
// chunks (the common case); the element-wise path is compiled separately so
// that it does not inflate the register budget of the chunked one.
template <bool kVec>
__global__ __launch_bounds__(256) void k_skinny(Launch L) {
  __shared__ __attribute__((aligned(16))) uint16_t As[64 * SLD];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[64 * SLD];
  const int pi = (L.nprob > 1 && (int)blockIdx.x >= L.p[1].wg_begin) ? 1 : 0;
  const Prob& P = L.p[pi];
  const SkinnyOp& op = P.op;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wi = wave >> 1, wj = wave & 1;
  const int local = (int)blockIdx.x - P.wg_begin;
  const int tile = local / P.splits, split = local % P.splits;
  const int64_t i0 = (int64_t)(tile / P.tiles_j) * 64, j0 = (int64_t)(tile % P.tiles_j) * 64;
  const int64_t cs = (int64_t)split * P.c_split;
  int64_t ce = cs + P.c_split;
  if (ce > op.C) ce = op.C;

  f32x16 acc = f32x16{};
  const int r32 = lane & 31, kh = (lane >> 5) * 8;
  OpRegs ra, rb;
  if (cs < ce) {
    load_op(ra, op.a, op.a_si, op.a_sc, i0, op.I, cs, ce, kVec || P.a_vec, tid);
    load_op(rb, op.b, op.b_sj, op.b_sc, j0, op.J, cs, ce, kVec || P.b_vec, tid);
  }
  for (int64_t c0 = cs; c0 < ce; c0 += kSkinnyStep) {
    store_op(As, ra, op.a_sc == 1, kVec || P.a_vec, tid);
    store_op(Bs, rb, op.b_sc == 1, kVec || P.b_vec, tid);
    __syncthreads();
    if (c0 + kSkinnyStep < ce) {  // next step's loads fly while this one computes
      load_op(ra, op.a, op.a_si, op.a_sc, i0, op.I, c0 + kSkinnyStep, ce, kVec || P.a_vec, tid);
      load_op(rb, op.b, op.b_sj, op.b_sc, j0, op.J, c0 + kSkinnyStep, ce, kVec || P.b_vec, tid);
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(As + (wi * 32 + r32) * SLD + kk * 16 + kh);
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(Bs + (wj * 32 + r32) * SLD + kk * 16 + kh);
      acc = mfma32(a, b, acc);
    }
    __syncthreads();
  }

  // Tile-local coordinates of this lane's accumulators.
  const int tj = wj * 32 + r32;
  if (P.splits == 1) {
    const int64_t j = j0 + tj;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t i = i0 + wi * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      if (i < op.I && j < op.J) put(P, i, j, acc[v]);
    }
    // Zero padding columns J <= j < Jw (only tiles in the last tile column).
    if (P.Jw > op.J && (tile % P.tiles_j) == P.tiles_j - 1) {
      for (int e = tid; e < 64 * (int)(P.Jw - op.J); e += 256) {
        const int64_t i = i0 + e / (P.Jw - op.J), j = op.J + e % (P.Jw - op.J);
        if (i < op.I) P.out[i * P.o_si + j] = 0;
      }
    }
  } else {
    float* mine = P.part + ((int64_t)tile * P.splits + split) * 4096;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int ti = wi * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      mine[ti * 64 + tj] = acc[v];
    }
  }
}

// ---------------------------------------------------------------------------
// Vectorized path (every operand aligned, contiguous extents multiples of 8).
// Each operand tile of a 64-deep step is staged in LDS in its natural layout
// (16-byte chunks along the operand's contiguous dimension): [x][c] when the
// contraction runs along memory, [c][x] when the output dimension does.  The
// MFMA fragments are read directly from the first and with the transposing
// LDS read (ds_read_b64_tr_b16) from the second, so no element is ever
// scattered.  Loads run three steps ahead in a register ring; every load is
// issued unconditionally (out-of-range chunks re-read the tile origin and
// are zeroed when stored), so the compiler waits only for the step consumed.
// ---------------------------------------------------------------------------
constexpr int kRing = 3;

struct VecSlot {
  u32x4 a[2], b[2];
};

// The two 16-byte chunks of one operand tile that a thread moves each step.
// Tile element (t, c) of natural row t: for a c-fast operand t is the output
// index and the columns are the contraction; otherwise t is the contraction
// index and the columns the output.  Chunk pointers advance by a fixed
// amount per step; a chunk is valid while its output index is in range and
// its contraction offset within the step is below the step's valid length.
struct VecOp {
  const uint16_t* ptr[2];  // chunk pointers at step 0 (the tile origin if out of range)
  const uint16_t* src;
  int64_t delta;           // per-step advance (elements)
  int coff[2];             // contraction offset of each chunk within a step
  bool xok[2];
};

template <bool kCFast>
__device__ __forceinline__ VecOp vec_op(const uint16_t* src, int64_t rstride, int64_t x0, int64_t X,
                                        int64_t cs, int tid) {
  VecOp o;
  o.src = src;
  o.delta = kCFast ? kSkinnyStep : kSkinnyStep * rstride;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int e = tid + 256 * q, r = e >> 3, cc = (e & 7) * 8;
    const int64_t x = kCFast ? x0 + r : x0 + cc;
    o.xok[q] = x < X;
    o.coff[q] = kCFast ? cc : r;
    o.ptr[q] = o.xok[q] ? src + (kCFast ? x * rstride + cs + cc : (cs + r) * rstride + x) : src;
  }
  return o;
}

// clen: valid contraction length of this step (0 .. 64)
__device__ __forceinline__ void vec_issue(u32x4 (&v)[2], const VecOp& o, int64_t step_off,
                                          int clen) {
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const bool ok = o.xok[q] & (o.coff[q] < clen);
    const uint16_t* pq = ok ? o.ptr[q] + step_off : o.src;
    v[q] = *reinterpret_cast<const u32x4*>(pq);
  }
}

__device__ __forceinline__ void vec_store(uint16_t* T, const u32x4 (&v)[2], const VecOp& o, int clen,
                                          int tid) {
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int e = tid + 256 * q;
    const bool ok = o.xok[q] & (o.coff[q] < clen);
    *reinterpret_cast<u32x4*>(T + (e >> 3) * SLD + (e & 7) * 8) = ok ? v[q] : u32x4{0u, 0u, 0u, 0u};
  }
}

// MFMA 32x32x16 fragment of sub-step kk: lane l gets output index base + l % 32
// and contraction rows 16 kk + 8 (l / 32) .. +7.
template <bool kCFast>
__device__ __forceinline__ bf16x8 vec_frag(const uint16_t* T, int base, int lane, int kk) {
  if (kCFast)
    return *reinterpret_cast<const bf16x8*>(T + (base + (lane & 31)) * SLD + kk * 16 + (lane >> 5) * 8);
  // [c][x]: within each 16-lane group g, lane i reads the 4-element chunk at
  // row 8 (g / 2) + i / 4 (+4 for the upper half), column 16 (g % 2) + 4 (i % 4)
  // and receives 4 consecutive rows of column i.
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
  const int g = lane >> 4, i = lane & 15;
  const int row = kk * 16 + 8 * (g >> 1) + (i >> 2);
  const int col = base + 16 * (g & 1) + 4 * (i & 3);
  const uint16_t* p0 = T + row * SLD + col;
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p0);
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p0 + 4 * SLD));
  const v8i16 v = v8i16{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

template <bool kACF, bool kBCF>
__device__ __forceinline__ void lora_vec_body(const Prob& P, int local,
                                              uint16_t (&Ts)[2][2][64 * SLD]) {
  const SkinnyOp op = P.op;
  const int splits = P.splits, tiles_j = P.tiles_j;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wi = wave >> 1, wj = wave & 1;
  const int tile = local / splits, split = local % splits;
  const int64_t i0 = (int64_t)(tile / tiles_j) * 64, j0 = (int64_t)(tile % tiles_j) * 64;
  const int64_t cs = (int64_t)split * P.c_split;
  int64_t ce = cs + P.c_split;
  if (ce > op.C) ce = op.C;
  // operand A (i, c) at a[i a_si + c a_sc], B (c, j) at b[j b_sj + c b_sc]
  const VecOp oa = vec_op<kACF>(op.a, kACF ? op.a_si : op.a_sc, i0, op.I, cs, tid);
  const VecOp ob = vec_op<kBCF>(op.b, kBCF ? op.b_sj : op.b_sc, j0, op.J, cs, tid);
  const int64_t nsteps = ce > cs ? (ce - cs + kSkinnyStep - 1) / kSkinnyStep : 0;

  VecSlot sl[kRing];
  // valid contraction length of step st (64 except on a ragged last step)
  auto step_len = [&](int64_t st) {
    const int64_t rem = ce - cs - st * kSkinnyStep;
    return rem >= kSkinnyStep ? kSkinnyStep : (int)rem;
  };
  auto issue = [&](VecSlot& S, int64_t st) {
    if (st >= nsteps) st = nsteps - 1;  // past the end: re-read the last step
    const int clen = step_len(st);
    vec_issue(S.a, oa, st * oa.delta, clen);
    vec_issue(S.b, ob, st * ob.delta, clen);
  };
  f32x16 acc = f32x16{};
  auto consume = [&](const VecSlot& S, int64_t st) {
    const int clen = step_len(st);
    uint16_t* TA = Ts[st & 1][0];
    uint16_t* TB = Ts[st & 1][1];
    vec_store(TA, S.a, oa, clen, tid);
    vec_store(TB, S.b, ob, clen, tid);
    // LDS writes visible to the workgroup; loads stay in flight
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const bf16x8 a = vec_frag<kACF>(TA, wi * 32, lane, kk);
      const bf16x8 b = vec_frag<kBCF>(TB, wj * 32, lane, kk);
      acc = mfma32(a, b, acc);
    }
  };

  if (nsteps > 0) {
#pragma unroll
    for (int u = 0; u < kRing - 1; ++u) issue(sl[u], u);
  }
  int64_t st = 0;
  for (; st + kRing <= nsteps; st += kRing) {
#pragma unroll
    for (int u = 0; u < kRing; ++u) {
      issue(sl[(u + kRing - 1) % kRing], st + u + kRing - 1);
      consume(sl[u], st + u);
    }
  }
#pragma unroll
  for (int u = 0; u < kRing - 1; ++u)
    if (st + u < nsteps) consume(sl[u], st + u);

  const int r32 = lane & 31;
  const int tj = wj * 32 + r32;
  if (splits == 1) {
    const int64_t j = j0 + tj;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t i = i0 + wi * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      if (i < op.I && j < op.J) put(P, i, j, acc[v]);
    }
    if (P.Jw > op.J && (tile % tiles_j) == tiles_j - 1) {
      for (int e = tid; e < 64 * (int)(P.Jw - op.J); e += 256) {
        const int64_t i = i0 + e / (P.Jw - op.J), j = op.J + e % (P.Jw - op.J);
        if (i < op.I) P.out[i * P.o_si + j] = 0;
      }
    }
  } else {
    float* mine = P.part + ((int64_t)tile * splits + split) * 4096;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int ti = wi * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      mine[ti * 64 + tj] = acc[v];
    }
  }
}

// Operand layouts of up to two products (c-fast A, c-fast B for each).
template <bool kA0, bool kB0, bool kA1, bool kB1>
__global__ __launch_bounds__(256) void k_lora_vec(Launch L) {
  __shared__ __attribute__((aligned(16))) uint16_t Ts[2][2][64 * SLD];  // [buffer][A, B]
  if (L.nprob > 1 && (int)blockIdx.x >= L.p[1].wg_begin)
    lora_vec_body<kA1, kB1>(L.p[1], (int)blockIdx.x - L.p[1].wg_begin, Ts);
  else
    lora_vec_body<kA0, kB0>(L.p[0], (int)blockIdx.x - L.p[0].wg_begin, Ts);
}

// Launch the vectorized kernel instance for the launch's operand layouts.
hipError_t launch_lora_vec(const Launch& L, int wg, hipStream_t stream) {
  auto cf = [&](int k, bool b) {
    const SkinnyOp& o = L.p[k < L.nprob ? k : 0].op;
    return b ? o.b_sc == 1 : o.a_sc == 1;
  };
  const int key = (cf(0, false) << 3) | (cf(0, true) << 2) | (cf(1, false) << 1) | cf(1, true);
  switch (key) {
#define QN_LORA_CASE(k)                                                                       \
  case k:                                                                                     \
    hipLaunchKernelGGL((k_lora_vec<(k >> 3) & 1, (k >> 2) & 1, (k >> 1) & 1, k & 1>),         \
                       dim3((unsigned)wg), dim3(256), 0, stream, L);                          \
    break;
    QN_LORA_CASE(0) QN_LORA_CASE(1) QN_LORA_CASE(2) QN_LORA_CASE(3)
    QN_LORA_CASE(4) QN_LORA_CASE(5) QN_LORA_CASE(6) QN_LORA_CASE(7)
    QN_LORA_CASE(8) QN_LORA_CASE(9) QN_LORA_CASE(10) QN_LORA_CASE(11)
    QN_LORA_CASE(12) QN_LORA_CASE(13) QN_LORA_CASE(14) QN_LORA_CASE(15)
#undef QN_LORA_CASE
  }
  return hipGetLastError();
}

// Second launch for products with several slices: four consecutive outputs
// of one tile row per thread; slices added in order.
__global__ __launch_bounds__(256) void k_skinny_finish(Launch L) {
  const int pi = (L.nprob > 1 && (int)blockIdx.x >= L.p[1].wg_begin) ? 1 : 0;
  const Prob& P = L.p[pi];
  const int64_t q = ((int64_t)blockIdx.x - P.wg_begin) * 256 + threadIdx.x;  // quad index
  const int64_t tile = q >> 10, off = (q & 1023) * 4;
  if (tile >= P.tiles) return;
  const f32x4* base = reinterpret_cast<const f32x4*>(P.part + tile * P.splits * 4096 + off);
  f32x4 s = base[0];
  for (int k = 1; k < P.splits; ++k) s += base[(int64_t)k * 1024];
  const int64_t i = (tile / P.tiles_j) * 64 + (off >> 6);
  const int64_t j = (tile % P.tiles_j) * 64 + (off & 63);
  if (i >= P.op.I) return;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (j + e < P.op.J) put(P, i, j + e, s[e]);
    else if (j + e < P.Jw) P.out[i * P.o_si + j + e] = 0;
  }
}


int64_t split_len(int64_t C, int s) {
  const int64_t steps = (C + kSkinnyStep - 1) / kSkinnyStep;
  return ((steps + s - 1) / s) * kSkinnyStep;
}

bool vec_ok(const uint16_t* ptr, int64_t sx, int64_t sc, int64_t X, int64_t C) {
  // 16-byte chunks need an aligned base and outer stride, a contraction
  // length that is a multiple of 8 and, for chunks along the output
  // dimension, an output extent that is a multiple of 8.
  const int64_t outer = (sc == 1) ? sx : sc;
  const bool along_x = (sc != 1);
  return ((uintptr_t)ptr & 15u) == 0 && (outer % 8) == 0 && (C % 8) == 0 &&
         (!along_x || (X % 8) == 0);
}

}  // namespace

int skinny_tiles(int64_t I, int64_t J) { return (int)(((I + 63) / 64) * ((J + 63) / 64)); }

int skinny_splits(int64_t I, int64_t J, int64_t C) {
  const int64_t tiles = skinny_tiles(I, J);
  const int64_t steps = (C + kSkinnyStep - 1) / kSkinnyStep;
  // About one workgroup per CU: more slices only add fp32 partial traffic
  // (written here, read by the finish launch), which costs more than the
  // extra overlap gains (measured with 256 to 2048 workgroups).
  int64_t s = (256 + tiles - 1) / tiles;
  const int64_t max_s = (steps + 7) / 8;   // keep >= 8 steps per slice
  if (s > max_s) s = max_s;
  if (s > 16) s = 16;
  if (s < 1) s = 1;
  return (int)s;
}

size_t skinny_partial_bytes(int64_t I, int64_t J, int64_t C) {
  const int s = skinny_splits(I, J, C);
  return s > 1 ? (size_t)skinny_tiles(I, J) * s * 4096 * sizeof(float) : 0;
}

SkinnyJob make_job(const SkinnyOp& op, float scale, uint16_t* out, int64_t o_si, int64_t Jw,
                   uint16_t* out2, int64_t o2_si, float* part) {
  SkinnyJob j;
  j.op = op;
  j.scale = scale;
  j.out = out;
  j.o_si = o_si;
  j.Jw = Jw;
  j.out2 = out2;
  j.o2_si = o2_si;
  j.part = part;
  return j;
}

hipError_t launch_skinny(const SkinnyJob* jobs, int njobs, hipStream_t stream) {
  Launch L{};
  L.nprob = njobs;
  int wg = 0;
  for (int k = 0; k < njobs; ++k) {
    const SkinnyJob& j = jobs[k];
    Prob& P = L.p[k];
    P.op = j.op;
    P.splits = skinny_splits(j.op.I, j.op.J, j.op.C);
    P.c_split = split_len(j.op.C, P.splits);
    P.scale = j.scale;
    P.out = j.out;
    P.o_si = j.o_si;
    P.Jw = j.Jw;
    P.out2 = j.out2;
    P.o2_si = j.o2_si;
    P.part = j.part;
    P.tiles_j = (int)((j.op.J + 63) / 64);
    P.tiles = skinny_tiles(j.op.I, j.op.J);
    P.wg_begin = wg;
    P.a_vec = vec_ok(j.op.a, j.op.a_si, j.op.a_sc, j.op.I, j.op.C);
    P.b_vec = vec_ok(j.op.b, j.op.b_sj, j.op.b_sc, j.op.J, j.op.C);
    wg += P.tiles * P.splits;
  }
  bool all_vec = true;
  for (int k = 0; k < njobs; ++k) all_vec = all_vec && L.p[k].a_vec && L.p[k].b_vec;
  hipError_t e;
  if (all_vec) {
    e = launch_lora_vec(L, wg, stream);
  } else {
    hipLaunchKernelGGL(k_skinny<false>, dim3((unsigned)wg), dim3(256), 0, stream, L);
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  // finish launch for the products with several slices: 4 quads of 1024 per tile
  Launch F{};
  int fwg = 0;
  for (int k = 0; k < njobs; ++k) {
    if (L.p[k].splits == 1) continue;
    F.p[F.nprob] = L.p[k];
    F.p[F.nprob].wg_begin = fwg;
    fwg += L.p[k].tiles * 4;
    ++F.nprob;
  }
  if (F.nprob == 0) return hipSuccess;
  hipLaunchKernelGGL(k_skinny_finish, dim3((unsigned)fwg), dim3(256), 0, stream, F);
  return hipGetLastError();
}


}  // namespace qn
