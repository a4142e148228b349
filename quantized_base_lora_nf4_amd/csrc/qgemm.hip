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
// Tiling (both kernels, default configuration): a 256 x 256 output tile per
// workgroup of 8 waves (2 x 4, two per SIMD), each wave owning 128 x 64
// outputs as 4 x 2 MFMA 32x32x16 tiles (128 fp32 accumulators per lane);
// 64-deep contraction steps; both operand tiles double-buffered in LDS
// (136 KiB) so that one barrier per step separates filling the next buffer
// from the MFMAs on the current one.
//
// Dequantization: each thread owns half of a 64-weight block row per step
// (a whole one with four waves).  It
// builds that block's 16 possible bf16 values, bf16_rne(level[i] * c_hat),
// once (16 multiplies), splits them into a low-byte and a high-byte plane of
// 4 registers each, and then resolves every code with byte permutes
// (v_perm_b32) in registers: no LDS lookups, and the tile is bit-identical to
// nf4_dequantize.
//
// Backward: the weight slice is written to LDS in its natural [n][k] layout
// and read as the MFMA B operand with ds_read_b64_tr_b16, which hands each
// lane 4 consecutive rows of one column.
#include <atomic>
#include <type_traits>

#include "kernels.hpp"

namespace qn {

namespace {

constexpr int BK = 64;    // contraction per step (one NF4 block)
constexpr int LDA = 72;   // LDS row stride (bf16) of [row][k] tiles: 64 + 8

// Workgroups are handed to the 8 XCDs round-robin by linear id, and each XCD
// has its own L2.  Remap so that each XCD receives a contiguous range of
// output tiles (tiles that share an operand tile then share an L2): linear
// id p runs on XCD p % 8, and becomes tile (p % 8) * (total / 8) + p / 8.
// The ids past the last full round of 8 keep their own index.
__device__ __forceinline__ int64_t xcd_tile(int64_t p, int64_t total) {
  const int64_t per = total >> 3;
  if (p >= per * 8) return p;
  return (p & 7) * per + (p >> 3);
}

__device__ __forceinline__ uint32_t perm(uint32_t s0, uint32_t s1, uint32_t sel) {
  return __builtin_amdgcn_perm(s0, s1, sel);
}

// Byte planes of the 16 candidate bf16 values of one block:
// lo[q] byte e = low byte of value 4q + e, hi[q] byte e = high byte.
struct LevelTable {
  uint32_t lo[4], hi[4];
};

template <class CT>
__device__ __forceinline__ LevelTable make_table(float chat, const UserTable& ut) {
  LevelTable t;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t p0 =
        pack_bf16x2(level_of<CT>(ut, 4 * q) * chat, level_of<CT>(ut, 4 * q + 1) * chat);
    const uint32_t p1 =
        pack_bf16x2(level_of<CT>(ut, 4 * q + 2) * chat, level_of<CT>(ut, 4 * q + 3) * chat);
    t.lo[q] = perm(p1, p0, 0x06040200u);
    t.hi[q] = perm(p1, p0, 0x07050301u);
  }
  return t;
}

// Eight codes (one 32-bit word; element order = nibble order) -> four packed
// bf16 pairs (element 2i in the low half of word i).
//   a, b: the codes of elements 0..3 and 4..7 spread one per byte, in order;
//   a byte select with selector c & 7 picks from the plane holding values
//   0..7 or 8..15, and a mask (0xFF where c >= 8) chooses between the two.
// The mask comes from v_perm's constant selectors on zero sources: selector
// c + 5 is a byte of zeros (5..7), a zero sign (8..11), 0x00 (12) or 0xFF
// (13 and above), so it is 0xFF exactly for c >= 8.
__device__ __forceinline__ u32x4 lookup8(uint32_t w, const LevelTable& t) {
  const uint32_t x = w & 0x0f0f0f0fu;          // elements 0, 2, 4, 6
  const uint32_t y = (w >> 4) & 0x0f0f0f0fu;   // elements 1, 3, 5, 7
  const uint32_t a = perm(y, x, 0x05010400u);  // elements 0, 1, 2, 3
  const uint32_t b = perm(y, x, 0x07030602u);  // elements 4, 5, 6, 7
  const uint32_t a7 = a & 0x07070707u, b7 = b & 0x07070707u;
  const uint32_t ma = perm(0u, 0u, a + 0x05050505u);
  const uint32_t mb = perm(0u, 0u, b + 0x05050505u);
  const uint32_t la = (ma & perm(t.lo[3], t.lo[2], a7)) | (~ma & perm(t.lo[1], t.lo[0], a7));
  const uint32_t ha = (ma & perm(t.hi[3], t.hi[2], a7)) | (~ma & perm(t.hi[1], t.hi[0], a7));
  const uint32_t lb = (mb & perm(t.lo[3], t.lo[2], b7)) | (~mb & perm(t.lo[1], t.lo[0], b7));
  const uint32_t hb = (mb & perm(t.hi[3], t.hi[2], b7)) | (~mb & perm(t.hi[1], t.hi[0], b7));
  return u32x4{perm(ha, la, 0x05010400u), perm(ha, la, 0x07030602u),
               perm(hb, lb, 0x05010400u), perm(hb, lb, 0x07030602u)};
}


// ---------------------------------------------------------------------------
// Tile configuration.  WM x WN waves, each owning FM x FN MFMA 32x32 tiles;
// workgroup tile BM x BN = (WM FM 32) x (WN FN 32); 64-deep steps.
// ---------------------------------------------------------------------------
template <int WM_, int WN_, int FM_, int FN_>
struct Cfg {
  static constexpr int WM = WM_, WN = WN_, FM = FM_, FN = FN_;
  static constexpr int NT = WM * WN * 64;           // threads
  static constexpr int BM = WM * FM * 32;           // output rows
  static constexpr int BN = WN * FN * 32;           // output columns
  static constexpr int TILE_A = BM * 64;            // [BM][64] activation tile (swizzled)
  static constexpr int TILE_BF = BN * LDA;          // forward weight tile [BN][LDA]
  static constexpr int BSTR = 72;                   // backward slice: stride of a 64-column block
  static constexpr int LDTB = (BN / 64) * BSTR;     // backward weight slice row stride
  static constexpr int TILE_BB = BK * LDTB;         // backward weight slice [64][LDTB]
  static constexpr int SMEM_F = 2 * (TILE_A + TILE_BF);
  static constexpr int SMEM_B = 2 * (TILE_A + TILE_BB);
  static constexpr int XCH = BM * 8 / NT;           // 16-byte activation chunks per thread
  static constexpr int XLD = BM / 8 / (NT / 64);    // direct-to-LDS loads per wave per step
  // Threads that expand weights: one whole block row (64 weights) each per
  // step, BN of them (the forward tile's BN rows; the backward slice's 64
  // rows x BN / 64 blocks).  With 8 waves these are waves 0-3; the other
  // four only run MFMAs, and each SIMD holds one wave of each kind.
  static constexpr int NDQ = BN;
  static_assert(SMEM_F * 2 <= 160 * 1024 && SMEM_B * 2 <= 160 * 1024, "LDS budget");
  static_assert(NDQ % 64 == 0 && NDQ <= NT, "whole waves expand weights");
};

// Activation tiles are [rows][64] bf16 with no padding; the eight 16-byte
// chunks of row r are stored in the order chunk ^ ((r >> 1) & 7), which keeps
// the MFMA fragment reads (16 consecutive rows, one chunk) free of LDS bank
// conflicts.  Offset (in elements) of chunk c of row r:
__device__ __forceinline__ int a_off(int r, int c) { return r * 64 + ((c ^ ((r >> 1) & 7)) << 3); }

// Direct global -> LDS load of a BM x 64 bf16 tile of a row-major matrix
// (row stride ld, columns c0..c0+63; rows past `rows` clamp to the last row,
// and a 16-byte chunk at or past column `cols` (a multiple of 8) re-reads
// column 0 of its row: the caller multiplies those columns by zero weights).
// Each wave instruction fills 8 consecutive tile rows (1 KB); lane l writes
// row 8 e + l / 8, slot l % 8, so it fetches the chunk that the swizzle puts
// in that slot.
//
// The loads use the buffer form (buffer_load_dwordx4 ... lds) through a
// resource whose base is the tile's first row.  With the global form the
// compiler treats every later wait as if a flat access were pending and
// drains all outstanding loads (vmcnt(0)) at the first use of any loaded
// register; with the buffer form its waits count only the loads that are
// actually needed, so the weight loads stay in flight across the step.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const uint16_t* src, int64_t ld,
                                                            int64_t row0, int64_t rows) {
  int64_t bytes = (rows - row0) * ld * 2;
  if (bytes > 0x7fffffff) bytes = 0x7fffffff;
  return __builtin_amdgcn_make_buffer_rsrc((void*)(src + row0 * ld), (short)0, (int)bytes,
                                           0x00020000);
}

template <class C, bool kClampCols>
__device__ __forceinline__ void load_rows_lds(uint16_t* As, __amdgpu_buffer_rsrc_t rsrc,
                                              int64_t ld, int64_t row0, int64_t rows, int64_t c0,
                                              int64_t cols, int wave, int lane) {
#pragma unroll
  for (int q = 0; q < C::XLD; ++q) {
    const int e = q * (C::NT / 64) + wave;  // 8-row group
    const int r = 8 * e + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    int64_t gr = row0 + r;
    if (gr >= rows) gr = rows - 1;
    // < 2^31 bytes: ld is at most 2^22 (the C ABI rejects larger N and K)
    if constexpr (kClampCols) {
      int64_t gc = c0 + c * 8;
      if (gc >= cols) gc = 0;
      const int voff = (int)(((gr - row0) * ld + gc) * 2);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsrc, (__attribute__((address_space(3))) void*)(As + 8 * e * 64), 16, voff, 0, 0, 0);
    } else {
      // the step's column offset is uniform: it goes in the scalar offset
      const int voff = (int)(((gr - row0) * ld + c * 8) * 2);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsrc, (__attribute__((address_space(3))) void*)(As + 8 * e * 64), 16, voff,
          (int)(c0 * 2), 0, 0);
    }
  }
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// End of a pipelined step: this wave's direct-to-LDS tile loads (issued
// first in the step) and LDS writes are complete, then the workgroup
// barrier.  The step's weight loads (issued after the tile loads) stay in
// flight into the next step, where they are consumed; vector memory loads
// complete in issue order, so vmcnt(kAfter) covers the tile loads when the
// step issued at least kAfter loads after them.
// The wait is issued through the builtin (s_waitcnt simm16: vmcnt in bits
// 3:0, expcnt 6:4, lgkmcnt 11:8) so that the compiler's own wait tracking
// knows the tile loads are complete; the empty asm statements keep memory
// operations from moving across it.
// kAfter must not exceed the number of load instructions the step issued
// after its tile loads (a smaller value only waits for more).
constexpr int kWLoads = 3;  // codes (at least one load), q8 byte, step
template <int kAfter = kWLoads>
__device__ __forceinline__ void step_barrier() {
  static_assert(kAfter >= 0 && kAfter <= 15, "vmcnt field");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0070 | kAfter);  // vmcnt(kAfter) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <class C>
struct AccT {
  f32x16 v[C::FM][C::FN];
};

template <class C>
__device__ __forceinline__ void zero_acc(AccT<C>& acc) {
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc.v[i][j] = f32x16{};
}

// MFMA operand fragments of one 16-deep sub-step.
template <class C>
struct Frags {
  bf16x8 a[C::FM], b[C::FN];
};

// Read the fragments of sub-step kk.  As: [BM][LDA] (rows = output rows, k
// contiguous).  B operand from Bs: forward [BN][LDA] (rows = output columns,
// k contiguous); backward [64][LDTB] (rows = k, columns = output columns in
// 64-column blocks of stride BSTR) read with the transposing LDS load.
template <class C, bool kTransB>
__device__ __forceinline__ void read_frags(Frags<C>& f, const uint16_t* As, const uint16_t* Bs,
                                           int wm, int wn, int lane, int kk) {
  const int r32 = lane & 31;
  const int kh = (lane >> 5) * 8;
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
    f.a[i] = *reinterpret_cast<const bf16x8*>(As + a_off(wm * C::FM * 32 + i * 32 + r32, 2 * kk + (kh >> 3)));
  if (!kTransB) {
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
      f.b[j] = *reinterpret_cast<const bf16x8*>(Bs + (wn * C::FN * 32 + j * 32 + r32) * LDA + kk * 16 + kh);
  } else {
    // Lane group g = lane / 16 covers columns 16 (g % 2) + 0..15 and
    // contraction rows 8 (g / 2) + 0..7; within the group, lane i reads the
    // 4-element chunk at row 4 h + i / 4, column 4 (i % 4) (h = 0, 1) and
    // receives 4 consecutive rows of column i.
    const int g = lane >> 4, i = lane & 15;
    const int row = kk * 16 + 8 * (g >> 1) + (i >> 2);
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
      typedef short v4i16 __attribute__((ext_vector_type(4)));
      typedef short v8i16 __attribute__((ext_vector_type(8)));
      typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
      const int col = wn * C::FN * 32 + j * 32 + 16 * (g & 1) + 4 * (i & 3);
      const uint16_t* p0 = Bs + row * C::LDTB + (col >> 6) * C::BSTR + (col & 63);
      const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p0);
      const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p0 + 4 * C::LDTB));
      const v8i16 v = v8i16{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      f.b[j] = __builtin_bit_cast(bf16x8, v);
    }
  }
}

template <class C>
__device__ __forceinline__ void mfma_frags(const Frags<C>& f, AccT<C>& acc) {
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc.v[i][j] = mfma32(f.a[i], f.b[j], acc.v[i][j]);
}

// A whole 64-deep step without other work (used for the LoRA steps and an
// odd last step).
template <class C, bool kTransB>
__device__ __forceinline__ void mma_step(const uint16_t* As, const uint16_t* Bs, int wm, int wn,
                                         int lane, AccT<C>& acc) {
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    Frags<C> f;
    read_frags<C, kTransB>(f, As, Bs, wm, wn, lane, kk);
    mfma_frags(f, acc);
  }
}

// Store the workgroup's accumulator tile as bf16 (row stride ld), skipping
// rows >= rows and columns >= cols.
template <class C>
__device__ __forceinline__ void store_tile(uint16_t* out, int64_t ld, int64_t row0, int64_t col0,
                                           int64_t rows, int64_t cols, int wm, int wn, int lane,
                                           const AccT<C>& acc) {
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
      const int64_t col = col0 + wn * C::FN * 32 + j * 32 + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = row0 + wm * C::FM * 32 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (row < rows && col < cols) out[row * ld + col] = f32_to_bf16(acc.v[i][j][v]);
      }
    }
}

// Stage a BM x 64 tile of a zero-padded bf16 matrix whose columns
// c0..c0+63 all exist (row stride a multiple of 8), scaling each element by
// `scale` in fp32 and rounding back to bf16 when do_scale is set.
template <class C>
__device__ __forceinline__ void stage_rows_scaled(uint16_t* As, const uint16_t* src, int64_t ld,
                                                  int64_t row0, int64_t rows, int64_t c0,
                                                  float scale, bool do_scale, int tid) {
#pragma unroll
  for (int q = 0; q < C::XCH; ++q) {
    const int e = tid + C::NT * q;
    const int row = e >> 3, c8 = e & 7;
    int64_t gr = row0 + row;
    if (gr >= rows) gr = rows - 1;
    u32x4 v = *reinterpret_cast<const u32x4*>(src + gr * ld + c0 + c8 * 8);
    if (do_scale) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        v[j] = pack_bf16x2(bf16_lo_to_f32(v[j]) * scale, bf16_hi_to_f32(v[j]) * scale);
    }
    *reinterpret_cast<u32x4*>(As + a_off(row, c8)) = v;
  }
}

// What one expanding thread loads for one contraction step: the codes of
// one whole block row (as two half-block word groups), its 8-bit constant
// and group step.
template <class CT>
struct StepRegs {
  HalfRaw<CT::kBits> c[2];
  uint32_t q;   // 8-bit constant as loaded
  float st;
};

template <class CT>
__device__ __forceinline__ void dequant_block(uint16_t* dst, const StepRegs<CT>& r,
                                              const UserTable& ut) {
  const LevelTable t = make_table<CT>((float)r.q * r.st, ut);
#pragma unroll
  for (int w = 0; w < 8; ++w)
    *reinterpret_cast<u32x4*>(dst + 8 * w) = lookup8(nibbles<CT>(r.c[w / 4], w % 4), t);
}

// One pipelined contraction step: the MFMAs on the current buffers (As, Bs)
// and, in an expanding thread (kD), the dequantized block row for the next
// step (codes loaded two steps earlier, in rn) written at Bw_n.  (The next
// activation tile is already on its way into the other buffer by
// direct-to-LDS loads.)  The four 16-deep sub-steps each read the next
// sub-step's fragments first, then run their MFMAs and the VALU work of
// expanding two code words, then write those weight chunks.  Expanding one
// whole block row per thread builds each block's table once (two threads
// on half rows built it twice), and pairing an expanding wave with an
// MFMA-only wave on each SIMD lets one's lookups run beside the other's
// MFMAs; measured 4-11 % faster than every wave expanding half rows.
template <class C, bool kTransB, class CT, bool kD>
__device__ __forceinline__ void step_interleaved(const uint16_t* As, const uint16_t* Bs,
                                                 uint16_t* Bw_n, const StepRegs<CT>& rn, int wm,
                                                 int wn, int lane, AccT<C>& acc,
                                                 const UserTable& ut) {
  Frags<C> f[2];
  read_frags<C, kTransB>(f[0], As, Bs, wm, wn, lane, 0);
  LevelTable t;
  if constexpr (kD) t = make_table<CT>((float)rn.q * rn.st, ut);
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    if (kk < 3) read_frags<C, kTransB>(f[(kk + 1) & 1], As, Bs, wm, wn, lane, kk + 1);
    mfma_frags(f[kk & 1], acc);
    if constexpr (kD) {
#pragma unroll
      for (int w = 2 * kk; w < 2 * kk + 2; ++w)
        *reinterpret_cast<u32x4*>(Bw_n + 8 * w) = lookup8(nibbles<CT>(rn.c[w / 4], w % 4), t);
    }
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
  UserTable ut;  // the caller's codebook (CodeUser types only)
};

// kQ4: K is a multiple of 256 (and q8 16-byte aligned, as the C ABI
// requires), so the constants of four consecutive blocks of a weight row are
// one aligned 32-bit word (and share one second-level step: 4 divides 256).  The row's constants are then
// loaded once per four steps instead of a byte and a float per step.
// BS: block size 64 << BS (one 8-bit constant per 64 << BS weights of a row;
// kQ4 only with BS = 0).
template <class C, class CT, bool kQ4, int BS>
__global__ __launch_bounds__(C::NT, 1) void k_qgemm_fwd(FwdArgs p) {
  static_assert(!kQ4 || BS == 0, "grouped constants need 64-element blocks");
  // One LDS object per buffer: the compiler's wait for a direct-to-LDS load
  // then applies only to reads of the buffer that load writes.
  __shared__ __attribute__((aligned(16))) uint16_t xs0[C::TILE_A];
  __shared__ __attribute__((aligned(16))) uint16_t xs1[C::TILE_A];
  __shared__ __attribute__((aligned(16))) uint16_t ws0[C::TILE_BF];
  __shared__ __attribute__((aligned(16))) uint16_t ws1[C::TILE_BF];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int64_t M = p.M, N = p.N, K = p.K;
  const int64_t tiles_n = (N + C::BN - 1) / C::BN;
  const int64_t tile = xcd_tile(blockIdx.x, tiles_n * ((M + C::BM - 1) / C::BM));
  const int64_t m0 = (tile / tiles_n) * C::BM, n0 = (tile % tiles_n) * C::BN;
  const int64_t kblocks = K >> 6;

  AccT<C> acc;
  zero_acc(acc);
  // Weight state through buffer resources (every offset below 2^31: the C
  // ABI keeps the codes under 2 GiB): a per-thread offset plus the step's
  // uniform offset, so the per-step address arithmetic is scalar.
  const __amdgpu_buffer_rsrc_t crs = bytes_rsrc(p.codes, N * kblocks * block_bytes<CT>());
  const int64_t cblocks = kblocks >> BS;  // constants per weight row
  const __amdgpu_buffer_rsrc_t qrs = bytes_rsrc(p.q8, N * cblocks);
  const __amdgpu_buffer_rsrc_t srs = bytes_rsrc(p.step, 4 * ((N * cblocks + 255) >> 8));
  const __amdgpu_buffer_rsrc_t xrsrc = rows_rsrc(p.X, K, m0, M);
  auto load_x = [&](uint16_t* As_dst, int64_t kt) {
    if (kt >= kblocks) kt = kblocks - 1;
    load_rows_lds<C, false>(As_dst, xrsrc, K, m0, M, kt * BK, K, wave, lane);  // K % 64 == 0
  };
  // The main loop, for an expanding thread (D: weight row tid of the tile,
  // clamped; rows past N are computed and dropped) or an MFMA-only one.
  // Both kinds pass the same barriers.
  auto run = [&](auto kind) {
    constexpr bool D = decltype(kind)::value;
    const int wrow = tid;
    int64_t gn = n0 + wrow;
    if (gn >= N) gn = N - 1;
    const int wvoff = (int)(gn * kblocks * block_bytes<CT>());
    const int64_t wblk0 = gn * cblocks;  // the row's first constant
    // Weights are loaded two steps ahead (two register sets) and expanded
    // into the other LDS buffer while the MFMAs of the current step run;
    // activations go straight from global memory into that buffer.  Steps
    // past the end reload the last step (harmless).
    StepRegs<CT> ra, rb;
    auto load_w = [&](StepRegs<CT>& r, int64_t kt) {
      if constexpr (D) {
        if (kt >= kblocks) kt = kblocks - 1;
#pragma unroll
        for (int h = 0; h < 2; ++h)
          r.c[h] = load_half<CT>(crs, wvoff + h * (int)half_bytes<CT>(),
                                 (int)(kt * block_bytes<CT>()));
        if constexpr (!kQ4) {
          // step kt lies in the row's constant kt >> BS
          r.q = __builtin_amdgcn_raw_buffer_load_b8(qrs, (int)wblk0, (int)(kt >> BS), 0);
          r.st = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                               srs, (int)(((wblk0 + (kt >> BS)) >> 8) * 4), 0, 0));
        }
      }
    };
    // kQ4: group g of four steps (4g .. 4g+3) keeps its constants in
    // register pair g % 2; group g + 1 is loaded when group g starts being
    // expanded.
    uint32_t q0 = 0, q1 = 0;
    float s0 = 0.0f, s1 = 0.0f;
    auto load_q4 = [&](uint32_t& q, float& st, int64_t g) {
      if constexpr (D) {
        if (g >= (kblocks >> 2)) g = (kblocks >> 2) - 1;
        q = __builtin_amdgcn_raw_buffer_load_b32(qrs, (int)wblk0, (int)(4 * g), 0);
        st = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                           srs, (int)(((wblk0 + 4 * g) >> 8) * 4), 0, 0));
      }
    };
    // One step: MFMAs on buffer `cur` for step kt, step kt + 1 expanded
    // into the other buffer.  kQ4: j = (kt + 1) % 4 is the position of step
    // kt + 1 in its group, whose constants are (qg, sg); j == 0 starts the
    // group and loads the next one into (ql, sl).  `last`: no later step
    // consumes this step's weight loads, so the compiler may drop them and
    // the barrier must wait for everything.
    auto body = [&](StepRegs<CT>& rnext, StepRegs<CT>& rload, int64_t kt, int cur, int j,
                    uint32_t& qg, float& sg, uint32_t& ql, float& sl, bool last) {
      const uint16_t* As = cur ? xs1 : xs0;
      const uint16_t* Bs = cur ? ws1 : ws0;
      uint16_t* As_n = cur ? xs0 : xs1;
      uint16_t* Bs_n = cur ? ws0 : ws1;
      load_x(As_n, kt + 1);   // tile loads first ...
      __builtin_amdgcn_sched_barrier(0);
      load_w(rload, kt + 2);  // ... then the weight loads, which outlive the step
      if constexpr (D && kQ4) {
        if (j == 0) load_q4(ql, sl, ((kt + 1) >> 2) + 1);
        rnext.q = (qg >> (8 * j)) & 0xffu;
        rnext.st = sg;
      }
      __builtin_amdgcn_sched_barrier(0);
      step_interleaved<C, false, CT, D>(As, Bs, Bs_n + wrow * LDA, rnext, wm, wn, lane, acc,
                                        p.ut);
      // loads after the tile loads: two code loads (>= 2 instructions),
      // plus q8 and step unless kQ4 (where a group start adds the word of
      // constants and the step); none in an MFMA-only thread
      if (last || !D)
        step_barrier<0>();
      else if (!kQ4 || j == 0)
        step_barrier<kWLoads>();
      else
        step_barrier<2>();
    };

    load_w(ra, 0);
    load_w(rb, 1);
    if constexpr (D && kQ4) {
      load_q4(q0, s0, 0);
      load_q4(q1, s1, 1);
      ra.q = q0 & 0xffu;
      ra.st = s0;
    }
    load_x(xs0, 0);
    if constexpr (D) dequant_block<CT>(ws0 + wrow * LDA, ra, p.ut);
    wait_vmem();
    __syncthreads();
    int64_t kt = 0;
    if constexpr (kQ4) {  // kblocks % 4 == 0; groups 2i and 2i + 1 per iteration
      for (; kt + 8 <= kblocks; kt += 8) {
        body(rb, ra, kt, 0, 1, q0, s0, q1, s1, false);
        body(ra, rb, kt + 1, 1, 2, q0, s0, q1, s1, false);
        body(rb, ra, kt + 2, 0, 3, q0, s0, q1, s1, false);
        body(ra, rb, kt + 3, 1, 0, q1, s1, q0, s0, false);
        body(rb, ra, kt + 4, 0, 1, q1, s1, q0, s0, false);
        body(ra, rb, kt + 5, 1, 2, q1, s1, q0, s0, false);
        body(rb, ra, kt + 6, 0, 3, q1, s1, q0, s0, false);
        body(ra, rb, kt + 7, 1, 0, q0, s0, q1, s1, false);
      }
      if (kt < kblocks) {  // one more group of four, the last steps
        body(rb, ra, kt, 0, 1, q0, s0, q1, s1, false);
        body(ra, rb, kt + 1, 1, 2, q0, s0, q1, s1, false);
        body(rb, ra, kt + 2, 0, 3, q0, s0, q1, s1, false);
        body(ra, rb, kt + 3, 1, 0, q1, s1, q0, s0, true);
        kt += 4;
      }
    } else {
      for (; kt + 2 <= kblocks; kt += 2) {
        // MFMA step kt (buffer 0), stage kt+1 from rb, load kt+2 into ra; then the converse
        body(rb, ra, kt, 0, 0, q0, s0, q1, s1, false);
        body(ra, rb, kt + 1, 1, 0, q0, s0, q1, s1, false);
      }
    }
    if (kt < kblocks) {  // odd number of steps: the last one is in buffer 0
      mma_step<C, false>(xs0, ws0, wm, wn, lane, acc);
      __syncthreads();
    }
  };
  if (tid < C::NDQ)  // whole waves
    run(std::true_type{});
  else
    run(std::false_type{});

  // LoRA: extra contraction over r with A-side bf16(s U) and B-side B.
  const bool bvec = (p.r & 7) == 0;
  for (int j0 = 0; j0 < p.r; j0 += 64) {
    uint16_t* As = xs0;
    uint16_t* Bs = ws0;
    stage_rows_scaled<C>(As, p.U, p.ldu, m0, M, j0, p.s, true, tid);
    for (int e = tid; e < C::BN * 8; e += C::NT) {
      const int row = e >> 3, c8 = e & 7;
      int64_t g = n0 + row;
      if (g >= N) g = N - 1;
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (bvec) {
        if (j0 + c8 * 8 < p.r) v = *reinterpret_cast<const u32x4*>(p.B + g * p.r + j0 + c8 * 8);
      } else {
        uint16_t t[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int jj = j0 + c8 * 8 + q;
          t[q] = (jj < p.r) ? p.B[g * p.r + jj] : (uint16_t)0;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = (uint32_t)t[2 * q] | ((uint32_t)t[2 * q + 1] << 16);
      }
      *reinterpret_cast<u32x4*>(Bs + row * LDA + c8 * 8) = v;
    }
    __syncthreads();
    mma_step<C, false>(As, Bs, wm, wn, lane, acc);
    __syncthreads();
  }

  store_tile<C>(p.Y, N, m0, n0, M, N, wm, wn, lane, acc);
}

// A per-thread buffer offset past every buffer this file reads (each under
// 2^31 bytes): such a load returns 0 without touching memory.
constexpr int kOutOfRange = INT32_MIN;

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
  UserTable ut;  // the caller's codebook (CodeUser types only)
};

// Output tile BM tokens x BN input features; contraction over the weight's
// rows in steps of 64.  The step's weight slice, rows n..n+63 and columns
// k0..k0+BN-1, is dequantized into Bs[64][LDTB] in its natural layout.
// BS: block size 64 << BS, as in the forward kernel.
template <class C, class CT, int BS>
__global__ __launch_bounds__(C::NT, 1) void k_qgemm_bwd(BwdArgs p) {
  __shared__ __attribute__((aligned(16))) uint16_t xs0[C::TILE_A];
  __shared__ __attribute__((aligned(16))) uint16_t xs1[C::TILE_A];
  __shared__ __attribute__((aligned(16))) uint16_t ws0[C::TILE_BB];
  __shared__ __attribute__((aligned(16))) uint16_t ws1[C::TILE_BB];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int64_t M = p.M, N = p.N, K = p.K;
  const int64_t tiles_k = (K + C::BN - 1) / C::BN;
  const int64_t tile = xcd_tile(blockIdx.x, tiles_k * ((M + C::BM - 1) / C::BM));
  const int64_t m0 = (tile / tiles_k) * C::BM, k0 = (tile % tiles_k) * C::BN;
  const int64_t kblocks = K >> 6;
  const int64_t nsteps = (N + BK - 1) / BK;

  AccT<C> acc;
  zero_acc(acc);
  // Weight state through buffer resources (offsets below 2^31 as in the
  // forward): a per-thread offset for weight row wr and block column kb_own
  // plus the step's uniform row offset.  A row past N (partial last step)
  // takes the per-thread offset 2^31, past every buffer's end whether or
  // not the range check counts the uniform offset: its loads return 0, so
  // its constant is 0 and its values +-0, and the dY columns it meets add
  // nothing.  Columns past K are computed from clamped codes and dropped
  // on store.  Every load is issued unconditionally.
  const int64_t rowb = kblocks * block_bytes<CT>();  // code bytes per weight row
  const __amdgpu_buffer_rsrc_t crs = bytes_rsrc(p.codes, N * rowb);
  const int64_t cblocks = kblocks >> BS;  // constants per weight row
  const __amdgpu_buffer_rsrc_t qrs = bytes_rsrc(p.q8, N * cblocks);
  const __amdgpu_buffer_rsrc_t srs = bytes_rsrc(p.step, 4 * ((N * cblocks + 255) >> 8));
  // dY tile of step ns straight into LDS; on a partial last step the chunks
  // past column N re-read column 0 and meet the zero rows above.
  const __amdgpu_buffer_rsrc_t yrsrc = rows_rsrc(p.dY, N, m0, M);
  auto load_x = [&](uint16_t* As_dst, int64_t ns) {
    if (ns >= nsteps) ns = nsteps - 1;
    load_rows_lds<C, true>(As_dst, yrsrc, N, m0, M, ns * BK, N, wave, lane);
  };
  // The main loop, for an expanding thread (D: weight slice row wr, block
  // column wb of the step's 64 x BN slice) or an MFMA-only one.  Both
  // kinds pass the same barriers.
  auto run = [&](auto kind) {
    constexpr bool D = decltype(kind)::value;
    constexpr int BPR = C::BN / 64;  // blocks per slice row
    const int wr = tid / BPR, wb = tid % BPR;
    const int64_t kcol = k0 + wb * 64;
    const int64_t kb_own = (kcol < K ? kcol : 0) >> 6;
    const int64_t qown = wr * cblocks + (kb_own >> BS);  // this thread's constant, row wr
    const int cvoff = (int)(wr * rowb + kb_own * block_bytes<CT>());
    StepRegs<CT> ra, rb;
    auto load_w = [&](StepRegs<CT>& r, int64_t ns) {
      if constexpr (D) {
        if (ns >= nsteps) ns = nsteps - 1;
        const int64_t srow = ns * BK;  // first weight row of the step
        const bool in = srow + wr < N;
#pragma unroll
        for (int h = 0; h < 2; ++h)
          r.c[h] = load_half<CT>(crs, in ? cvoff + h * (int)half_bytes<CT>() : kOutOfRange,
                                 (int)(srow * rowb));
        r.q = __builtin_amdgcn_raw_buffer_load_b8(qrs, in ? (int)qown : kOutOfRange,
                                                  (int)(srow * cblocks), 0);
        r.st = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(
                       srs, in ? (int)(((srow * cblocks + qown) >> 8) * 4) : kOutOfRange, 0, 0));
      }
    };
    auto body = [&](StepRegs<CT>& rnext, StepRegs<CT>& rload, int64_t ns, int cur) {
      const uint16_t* As = cur ? xs1 : xs0;
      const uint16_t* Bs = cur ? ws1 : ws0;
      uint16_t* As_n = cur ? xs0 : xs1;
      uint16_t* Bs_n = cur ? ws0 : ws1;
      load_x(As_n, ns + 1);    // tile loads first ...
      __builtin_amdgcn_sched_barrier(0);
      load_w(rload, ns + 2);   // ... then the weight loads, which outlive the step
      __builtin_amdgcn_sched_barrier(0);
      step_interleaved<C, true, CT, D>(As, Bs, Bs_n + wr * C::LDTB + wb * C::BSTR, rnext, wm,
                                       wn, lane, acc, p.ut);
      // two code loads, q8 and step after the tile loads (>= kWLoads); none
      // in an MFMA-only thread
      if constexpr (D)
        step_barrier<kWLoads>();
      else
        step_barrier<0>();
    };

    load_w(ra, 0);
    load_w(rb, 1);
    load_x(xs0, 0);
    if constexpr (D) dequant_block<CT>(ws0 + wr * C::LDTB + wb * C::BSTR, ra, p.ut);
    wait_vmem();
    __syncthreads();
    int64_t ns = 0;
    for (; ns + 2 <= nsteps; ns += 2) {
      body(rb, ra, ns, 0);
      body(ra, rb, ns + 1, 1);
    }
    if (ns < nsteps) {
      mma_step<C, true>(xs0, ws0, wm, wn, lane, acc);
      __syncthreads();
    }
  };
  if (tid < C::NDQ)  // whole waves
    run(std::true_type{});
  else
    run(std::false_type{});

  // LoRA: dX += dU A, contraction over r.  A[j][k] is already [contraction][column].
  for (int j0 = 0; j0 < p.r; j0 += 64) {
    uint16_t* As = xs0;
    uint16_t* Bs = ws0;
    stage_rows_scaled<C>(As, p.dU, p.lddu, m0, M, j0, 1.0f, false, tid);
    for (int e = tid; e < 64 * (C::BN / 8); e += C::NT) {
      const int jr = e / (C::BN / 8), c8 = e % (C::BN / 8);  // adapter row j0 + jr
      const int64_t col = k0 + c8 * 8;
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (j0 + jr < p.r && col < K) v = *reinterpret_cast<const u32x4*>(p.A + (j0 + jr) * K + col);
      *reinterpret_cast<u32x4*>(Bs + jr * C::LDTB + (c8 >> 3) * C::BSTR + (c8 & 7) * 8) = v;
    }
    __syncthreads();
    mma_step<C, true>(As, Bs, wm, wn, lane, acc);
    __syncthreads();
  }

  store_tile<C>(p.dX, K, m0, k0, M, K, wm, wn, lane, acc);
}

#ifndef QN_GEMM_CFG
#define QN_GEMM_CFG 2, 4, 4, 2
#endif
using GemmCfg = Cfg<QN_GEMM_CFG>;
// 128 x 128 tiles, the same 8 waves (each 64 x 32): for grids the 256 x 256
// tiles would leave mostly idle (few tokens times a narrow weight), where
// four times as many workgroups still run in at most two passes over the CUs.
using SmallCfg = Cfg<2, 4, 2, 1>;

// Compute units of the current device (the one the launch goes to), asked
// once per device; 0 if the query fails, which keeps the large tiles.
int device_cus() {
  static std::atomic<int> known[64];
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < 64 && (cus = known[dev].load(std::memory_order_relaxed)) > 0) return cus;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  if (dev >= 0 && dev < 64) known[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// The small tiles when the 256 x 256 grid of an M x cols output fills at
// most half the compute units.
bool small_tiles(int64_t M, int64_t cols) {
  const int64_t big = ((M + GemmCfg::BM - 1) / GemmCfg::BM) * ((cols + GemmCfg::BN - 1) / GemmCfg::BN);
  return 2 * big <= device_cus();
}

template <class C>
hipError_t launch_fwd(const FwdArgs& a, const Nf4View& w, int64_t M, hipStream_t stream) {
  dim3 grid((unsigned)(((w.N + C::BN - 1) / C::BN) * ((M + C::BM - 1) / C::BM)));
  const bool q4 = (w.K % 256) == 0 && w.bshift == 0;
  with_any_code(w.code, [&](auto ct) {
    using CT = decltype(ct);
    if (q4)
      hipLaunchKernelGGL((k_qgemm_fwd<C, CT, true, 0>), grid, dim3(C::NT), 0, stream, a);
    else if (w.bshift == 2)
      hipLaunchKernelGGL((k_qgemm_fwd<C, CT, false, 2>), grid, dim3(C::NT), 0, stream, a);
    else if (w.bshift == 1)
      hipLaunchKernelGGL((k_qgemm_fwd<C, CT, false, 1>), grid, dim3(C::NT), 0, stream, a);
    else
      hipLaunchKernelGGL((k_qgemm_fwd<C, CT, false, 0>), grid, dim3(C::NT), 0, stream, a);
    return 0;
  });
  return hipGetLastError();
}

template <class C>
hipError_t launch_bwd(const BwdArgs& a, const Nf4View& w, int64_t M, hipStream_t stream) {
  dim3 grid((unsigned)(((w.K + C::BN - 1) / C::BN) * ((M + C::BM - 1) / C::BM)));
  with_any_code(w.code, [&](auto ct) {
    using CT = decltype(ct);
    if (w.bshift == 2)
      hipLaunchKernelGGL((k_qgemm_bwd<C, CT, 2>), grid, dim3(C::NT), 0, stream, a);
    else if (w.bshift == 1)
      hipLaunchKernelGGL((k_qgemm_bwd<C, CT, 1>), grid, dim3(C::NT), 0, stream, a);
    else
      hipLaunchKernelGGL((k_qgemm_bwd<C, CT, 0>), grid, dim3(C::NT), 0, stream, a);
    return 0;
  });
  return hipGetLastError();
}

}  // namespace

hipError_t launch_qgemm_fwd(const Nf4View& w, const uint16_t* X, int64_t M, const uint16_t* U,
                            int64_t ldu, const uint16_t* B, int32_t r, float s, uint16_t* Y,
                            hipStream_t stream) {
  const FwdArgs a{X, w.codes, w.q8, w.step, U, ldu, B, r, s, Y, M, w.N, w.K, w.ut};
  return small_tiles(M, w.N) ? launch_fwd<SmallCfg>(a, w, M, stream)
                             : launch_fwd<GemmCfg>(a, w, M, stream);
}

hipError_t launch_qgemm_bwd(const Nf4View& w, const uint16_t* dY, int64_t M, const uint16_t* dU,
                            int64_t lddu, const uint16_t* A, int32_t r, uint16_t* dX,
                            hipStream_t stream) {
  const BwdArgs a{dY, w.codes, w.q8, w.step, dU, lddu, A, r, dX, M, w.N, w.K, w.ut};
  return small_tiles(M, w.K) ? launch_bwd<SmallCfg>(a, w, M, stream)
                             : launch_bwd<GemmCfg>(a, w, M, stream);
}

}  // namespace qn
