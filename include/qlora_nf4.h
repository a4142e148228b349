/*
 * qlora_nf4.h -- C ABI of the frozen-NF4-base + LoRA linear layer for
 * AMD Instinct MI355X (gfx950).
 *
 * What the layer is (cited by page title and section):
 *  - The frozen base weight is stored in 4-bit NormalFloat (NF4): 16 levels
 *    at normal quantiles, one absmax scaling constant per block of weights,
 *    and the constants themselves quantized to 8 bits under a coarser set of
 *    constants ("QLoRA: fine-tuning a 65B model on one GPU", section
 *    "NormalFloat, double quantization, paged optimizers"; "QLoRA: efficient
 *    finetuning of quantized LLMs", Abstract, items (a) and (b)).
 *  - The base is quantized once up front and dequantized to 16 bits on the
 *    fly for every forward and backward pass; gradients reach only the
 *    low-rank adapters, which stay in 16 bits (blog section "Where the memory
 *    goes"; CoChat Abstract).
 *  - The backward pass re-materializes the low-precision weight from the
 *    quantized module instead of keeping a 16-bit copy ("ModuLoRA: Finetuning
 *    2-Bit LLMs on Consumer GPUs by Integrating with Modular Quantizers",
 *    abstract).
 *
 * Shapes (torch Linear convention, row-major, contiguous):
 *   W [N, K]  frozen weight (fp32 only as quantizer input)
 *   X [M, K]  input, bf16            Y  [M, N] output, bf16
 *   A [r, K]  LoRA down, bf16        B  [N, r] LoRA up, bf16
 *   s         LoRA scale (alpha / r), fp32
 *   Forward:  Y  = X W^T + s (X A^T) B^T
 *   Backward: dU = s dY B;  dX = dY W + dU A;  dA = dU^T X;  dB = s dY^T (X A^T)
 *   where W is the dequantized weight; there is no gradient for W.
 *
 * NF4 storage of W (the "nf4 tensor"), block size B = 64 by default (128
 * and 256 are offered too: the LQ-LoRA abstract's integer program chooses
 * the block size per matrix):
 *   codes [N*K/2] uint8  two 4-bit level indices per byte, element 2j of the
 *                        row-major flattening in the low nibble of byte j
 *   q8    [N*K/B] uint8  8-bit absmax constant of each B-element block
 *   step  [ceil(N*K/B/256)] fp32  per group of 256 consecutive blocks:
 *                        the group's largest absmax divided by 255
 *   Dequantized weight: w = bf16_rne(level[code] * (q8 * step)), both
 *   products rounded to fp32.
 *
 * Code types (the table `level[16]` behind the 4-bit codes; the capability
 * page "Qlora 4 Bit Quantization With Nf4 Fp4 Data Types And Lora Adapters"
 * names both data types, and the blog section "NormalFloat, double
 * quantization, paged optimizers" compares NF4 against a plain 4-bit float):
 *   QLORA_CODE_NF4  the 16 NF4 levels, ascending with the code, zero = code 7
 *   QLORA_CODE_FP4  4-bit float E2M1 read as: bit 3 sign, bits 2..1 exponent
 *                   (bias 1, exponent 0 subnormal), bit 0 mantissa, i.e.
 *                   magnitudes {0, 1/2, 1, 3/2, 2, 3, 4, 6}, divided by 6
 *                   so the largest is 1, rounded once to fp32; code 8 is -0
 *                   and the quantizer writes code 0 for zero.
 *   QLORA_CODE_NF3, QLORA_CODE_NF2  k-bit NormalFloat, k = 3, 2 (the
 *                   "ModuLoRA: Finetuning 2-Bit LLMs on Consumer GPUs by
 *                   Integrating with Modular Quantizers" abstract finetunes
 *                   through 2-, 3- and 4-bit weights): 2^k levels built as
 *                   NF4's are (exact zero, 2^(k-1) positive and 2^(k-1)-1
 *                   negative levels at evenly spaced normal probabilities
 *                   up to delta_k = 1 - (1/(2(2^k-1)) + 1/2^(k+1))/2, over
 *                   Phi^{-1}(delta_k)); ascending with the code.
 *   QLORA_CODE_USER4, QLORA_CODE_USER3, QLORA_CODE_USER2  a caller's
 *                   codebook of 2^k values, k = 4, 3, 2 (the ModuLoRA
 *                   abstract materializes the low-precision weight from a
 *                   black-box quantizer: the kernels only need the values
 *                   behind the codes).  The values, fp32 in code order, are
 *                   passed in nf4_tensor_t.levels (and to
 *                   qlora_quantize_user); each must be finite with
 *                   |v| <= 1, and either 0 or |v| >= 2^-20 (so that every
 *                   midpoint of two values is exact in fp64); any order,
 *                   repeats allowed.  Quantizer: the nearest value, ties to
 *                   the lower value, of equal values the lowest code; an
 *                   all-zero block takes the code of the value nearest to 0.
 *                   Accepted by the quantizer, the dequantizer and the
 *                   layer; not by qlora_lq_init and the configuration-error
 *                   calls (QLORA_ERR_UNSUPPORTED).
 *   Block scaling and double quantization are the same for all types.
 *
 * Code storage by width k (4 for NF4 and FP4): a 64-element block takes
 * 8k bytes, two halves of 4k bytes (k little-endian 32-bit words) for
 * elements 0..31 and 32..63.  k = 4: the layout above (element 2j of the
 * block in the low nibble of byte j).  k = 3, 2: within a half, element
 * 8g + 2i + p (g, i in 0..3, p in 0..1) keeps code bits 0-1 at bit 8i + 2g
 * of word p and, for k = 3, code bit 2 at bit (8i + 2 + 2g + p) mod 32 of
 * word 2.  `codes` then holds N*K*k/8 bytes.
 *
 * Conventions for every call:
 *   - bf16 tensors are passed as uint16_t bit patterns.
 *   - All tensor pointers are DEVICE pointers owned by the caller; the
 *     library never allocates, frees or keeps them.  Scratch memory comes
 *     from a caller-provided device workspace sized by
 *     qlora_workspace_size().  Pointers must be 16-byte aligned.
 *   - Work is enqueued on `stream` (0 = the null stream) and is
 *     asynchronous; no call synchronizes.  Apart from the fixed scratch
 *     array of qlora_linear_fwd_noalloc (below), the library keeps no
 *     mutable global state: calls are reentrant and thread-safe.  Calls that
 *     share a workspace must be ordered (same stream).
 *   - Every call validates its arguments before launching anything and
 *     returns a status code (QLORA_OK or a negative error, see below).  On
 *     an argument error (QLORA_ERR_INVALID, _UNSUPPORTED, _WORKSPACE)
 *     nothing has been enqueued and no output has been touched.
 *     QLORA_ERR_LAUNCH means a launch failed after the arguments were
 *     accepted: launches of the same call made before it stay enqueued, and
 *     the outputs are undefined.
 *   - Results are deterministic: the same inputs give bit-identical outputs.
 */
#ifndef QLORA_NF4_H_
#define QLORA_NF4_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---- */
#define QLORA_OK 0
#define QLORA_ERR_INVALID (-1)     /* null pointer, bad size, misalignment   */
#define QLORA_ERR_UNSUPPORTED (-2) /* block sizes other than 64 / 256, etc.  */
#define QLORA_ERR_WORKSPACE (-3)   /* workspace smaller than required        */
#define QLORA_ERR_LAUNCH (-4)      /* a HIP launch reported an error         */
#define QLORA_ERR_INFEASIBLE (-5)  /* qlora_ilp_plan: no choice fits          */

#define QLORA_CODE_NF4 0
#define QLORA_CODE_FP4 1
#define QLORA_CODE_NF3 2
#define QLORA_CODE_NF2 3
#define QLORA_CODE_USER4 4
#define QLORA_CODE_USER3 5
#define QLORA_CODE_USER2 6
/* Smallest magnitude of a nonzero value of a caller's codebook: 2^-20. */
#define QLORA_USER_MIN_MAGNITUDE (1.0f / 1048576.0f)

#define QLORA_NF4_BLOCKSIZE 64
#define QLORA_NF4_DQ_BLOCKSIZE 256
#define QLORA_MAX_RANK 256
/* Largest N and K accepted by qlora_linear_fwd / qlora_linear_bwd (a 256-row
 * tile of X or dY must span less than 2 GiB). */
#define QLORA_LINEAR_MAX_NK (1 << 22)

/* The quantized frozen weight.  All pointers are device pointers. */
typedef struct nf4_tensor_t {
  const uint8_t* codes; /* [N*K*k/8], k = bits of code_type */
  const uint8_t* q8;    /* [N*K/blocksize] */
  const float* step;    /* [ceil(N*K/blocksize/256)] */
  int64_t N;
  int64_t K;
  int32_t blocksize;    /* 64, 128 or 256, dividing K (others give
                           QLORA_ERR_UNSUPPORTED; K not a multiple of it,
                           QLORA_ERR_INVALID) */
  int32_t dq_blocksize; /* must be 256 */
  int32_t code_type;    /* QLORA_CODE_* (the type it was quantized with);
                           others give QLORA_ERR_UNSUPPORTED */
  const float* levels;  /* QLORA_CODE_USER*: HOST pointer to the 2^k code
                           values (code order), read during each call that
                           takes the tensor and not kept; NULL or values
                           outside the contract give QLORA_ERR_INVALID.
                           Ignored for the built-in code types. */
} nf4_tensor_t;

/* Text for a status code (static storage, never NULL). */
const char* qlora_status_str(int32_t status);

/* Host-side copy of the 16 NF4 levels (ascending, fp32) and of the 15
 * decision thresholds the quantizer compares against (a value x normalized
 * by its block's absmax gets the code #{i : x > thresholds[i]}, which is the
 * nearest level with ties going to the lower one).  No device work.  Either
 * pointer may be NULL.  Levels: normal quantiles with an exact zero,
 * normalized to [-1, 1] ("QLoRA: fine-tuning a 65B model on one GPU",
 * section "NormalFloat, double quantization, paged optimizers"). */
void nf4_code_table(float* levels16, float* thresholds15);

/* Host-side copy of the value of each code of `code_type` (in code order,
 * fp32; entries past 2^k are 0) and of its decision thresholds: the fp32
 * midpoint of each pair of consecutive distinct values, rounded toward
 * -inf, ascending (NF4: 15; FP4: 14, since +0 and -0 are one value; NF3: 7;
 * NF2: 3; the rest of thresholds15 is set to 0).  Returns the number of
 * thresholds, or QLORA_ERR_UNSUPPORTED for an unknown code type.  Either
 * pointer may be NULL; no device work. */
int32_t qlora_code_table(int32_t code_type, float* levels16, float* thresholds15);

/* Host-side check of a caller's codebook for QLORA_CODE_USER* and the
 * decision thresholds the quantizer derives from it (as qlora_code_table
 * gives them for the built-in types: the fp32 midpoint of each pair of
 * consecutive distinct values, rounded toward -inf, ascending; the rest of
 * thresholds15 is set to 0).  levels: 2^k fp32 values (host).  Returns the
 * number of thresholds, QLORA_ERR_UNSUPPORTED for a code type that is not a
 * user type, or QLORA_ERR_INVALID for NULL levels or values outside the
 * contract.  thresholds15 may be NULL; no device work. */
int32_t qlora_user_table(int32_t code_type, const float* levels, float* thresholds15);

/* Bytes of the three arrays of one configuration (code type, block size 64,
 * 128 or 256) for an N x K weight: N*K*k/8 + N*K/B + 4*ceil(N*K/B/256), k
 * the code width and B the block size; 0 for invalid sizes, an unknown code
 * type or an unsupported block size. */
size_t qlora_config_bytes(int32_t code_type, int32_t blocksize, int64_t N, int64_t K);

/* Bytes of the three NF4 arrays for an N x K weight (closed form:
 * N*K/2 + N*K/64 + 4*ceil(N*K/16384)); 0 for invalid sizes. */
size_t nf4_storage_bytes(int64_t N, int64_t K);

/* The same for any code type: N*K*k/8 + N*K/64 + 4*ceil(N*K/16384) with k
 * its width in bits; 0 for invalid sizes or an unknown code type. */
size_t qlora_storage_bytes(int32_t code_type, int64_t N, int64_t K);

/* nf4_quantize -- blockwise NF4 quantization with double-quantized absmax
 * constants, once per frozen weight (blog section "NormalFloat, double
 * quantization, paged optimizers"; capability page "Qlora 4 Bit
 * Quantization With Nf4 Fp4 Data Types And Lora Adapters", NF4 entry:
 * block-wise absmax scaling and double quantization of the constants).
 *
 *   W      [N, K] fp32, device.  Must be finite.
 *   N, K   N >= 1, K >= 64, K % 64 == 0.
 *   blocksize, dq_blocksize   64, 128 or 256 (dividing K), and 256; codes
 *          are packed in 64-element units whatever the block size, q8 has
 *          N*K/blocksize bytes and step ceil(N*K/blocksize/256) floats.
 *   codes  [N*K/2] out;  q8 [N*K/64] out;  step [ceil(N*K/16384)] out.
 * Per block b of 64 consecutive elements: c_b = max|w|; each element gets
 * the level nearest to fl32(w / c_b) (ties to the lower level; an all-zero
 * block gets the zero level).  Per group g of 256 consecutive blocks (the
 * last group may be shorter): step_g = fl32(max_b c_b / 255),
 * q_b = min(255, round_half_even(fl32(c_b / step_g))), q_b = 0 if step_g = 0.
 */
int32_t nf4_quantize(const float* W, int64_t N, int64_t K, int32_t blocksize,
                     int32_t dq_blocksize, uint8_t* codes, uint8_t* q8,
                     float* step, hipStream_t stream);

/* qlora_quantize -- nf4_quantize for any code type: identical except that
 * each element gets the code of the value of `code_type` nearest to
 * fl32(w / c_b) (ties to the lower value; zero, and an all-zero block, get
 * the code of zero: 7 for NF4, 0 for FP4, 3 for NF3, 1 for NF2), stored at
 * the type's width (codes [N*K*k/8]).  An unknown code type gives
 * QLORA_ERR_UNSUPPORTED, a user code type QLORA_ERR_INVALID (it needs its
 * values: qlora_quantize_user).  nf4_quantize(...) is
 * qlora_quantize(..., QLORA_CODE_NF4, ...). */
int32_t qlora_quantize(const float* W, int64_t N, int64_t K, int32_t code_type,
                       int32_t blocksize, int32_t dq_blocksize, uint8_t* codes,
                       uint8_t* q8, float* step, hipStream_t stream);

/* qlora_quantize_user -- qlora_quantize with a caller's codebook:
 * code_type QLORA_CODE_USER4, _USER3 or _USER2 and `levels` (host, 2^k
 * fp32 values in code order, read during the call) under the contract and
 * quantizer rule above.  The division w / c_b is the IEEE-correct one for
 * every block.  A built-in code type gives QLORA_ERR_UNSUPPORTED (use
 * qlora_quantize); bad levels, QLORA_ERR_INVALID. */
int32_t qlora_quantize_user(const float* W, int64_t N, int64_t K, int32_t code_type,
                            const float* levels, int32_t blocksize, int32_t dq_blocksize,
                            uint8_t* codes, uint8_t* q8, float* step, hipStream_t stream);

/* nf4_dequantize -- materialize the bf16 weight [N, K] from its quantized
 * state, with the code table of w->code_type (for checking and interop; the
 * linear layer never does this: it dequantizes tiles on chip).  w->N, w->K
 * as in nf4_quantize.  W_bf16 [N*K] out. */
int32_t nf4_dequantize(const nf4_tensor_t* w, uint16_t* W_bf16,
                       hipStream_t stream);

/* Workspace bytes needed by qlora_linear_fwd (for_bwd = 0) or
 * qlora_linear_bwd (for_bwd = 1) at these sizes; 0 for invalid sizes. */
size_t qlora_workspace_size(int64_t M, int64_t N, int64_t K, int32_t r,
                            int32_t for_bwd);

/* qlora_linear_fwd -- Y = X W^T + s (X A^T) B^T with W dequantized on the
 * fly to bf16 (blog section "Where the memory goes").
 *
 *   w       quantized weight, N >= 1, N % 8 == 0, K % 64 == 0,
 *           N, K <= QLORA_LINEAR_MAX_NK, packed codes under 2 GiB
 *           (N K bits / 8 < 2^31)
 *   X       [M, K] bf16, M >= 1
 *   A       [r, K] bf16;  B [N, r] bf16;  1 <= r <= 256
 *   s       LoRA scale
 *   Y       [M, N] bf16 out
 *   U_out   [M, r] bf16 out, may be NULL: X A^T rounded to bf16, which
 *           qlora_linear_bwd can take back instead of recomputing it
 *   ws      device workspace of ws_bytes >= qlora_workspace_size(M,N,K,r,0)
 * Accumulation is fp32.  M <= 16 takes a bandwidth-bound path that
 * streams the packed weight once (when its per-workgroup tables fit in
 * LDS: K up to about 32000 at M = 16, r = 256); larger M, or
 * larger K, takes the MFMA tile path.  Both meet the same tolerance.
 */
int32_t qlora_linear_fwd(const nf4_tensor_t* w, const uint16_t* X, int64_t M,
                         const uint16_t* A, const uint16_t* B, int32_t r,
                         float s, uint16_t* Y, uint16_t* U_out, void* ws,
                         size_t ws_bytes, hipStream_t stream);

/* qlora_linear_bwd -- gradients of the layer for the output gradient dY,
 * re-dequantizing W on chip (ModuLoRA abstract: the backward pass
 * materializes the low-precision weight from the quantized module):
 *   dX = dY W + s (dY B) A      [M, K] bf16 out, may be NULL (skipped)
 *   dA = s (dY B)^T X           [r, K] bf16 out
 *   dB = s dY^T (X A^T)         [N, r] bf16 out
 * Outputs are overwritten, not accumulated.  U is X A^T as returned by
 * qlora_linear_fwd's U_out, or NULL to recompute it.  Other arguments as in
 * qlora_linear_fwd; ws_bytes >= qlora_workspace_size(M,N,K,r,1).
 */
int32_t qlora_linear_bwd(const nf4_tensor_t* w, const uint16_t* X,
                         const uint16_t* dY, int64_t M, const uint16_t* A,
                         const uint16_t* B, const uint16_t* U, int32_t r,
                         float s, uint16_t* dX, uint16_t* dA, uint16_t* dB,
                         void* ws, size_t ws_bytes, hipStream_t stream);

/* Measurement variants of the two layer calls: identical work, and in
 * addition `ev_begin` is recorded on `stream` right before, and `ev_end`
 * right after, the launch of the dequantizing main kernel (the MFMA tile
 * GEMM, or for M <= 16 in the forward pass the weight-streaming kernel; in
 * the backward pass the dX GEMM, so nothing is recorded when dX is NULL).
 * hipEventElapsedTime over the pair is that kernel's duration.  Either
 * event may be NULL.  The events are created and owned by the caller. */
int32_t qlora_linear_fwd_ev(const nf4_tensor_t* w, const uint16_t* X,
                            int64_t M, const uint16_t* A, const uint16_t* B,
                            int32_t r, float s, uint16_t* Y, uint16_t* U_out,
                            void* ws, size_t ws_bytes, hipStream_t stream,
                            hipEvent_t ev_begin, hipEvent_t ev_end);
int32_t qlora_linear_bwd_ev(const nf4_tensor_t* w, const uint16_t* X,
                            const uint16_t* dY, int64_t M, const uint16_t* A,
                            const uint16_t* B, const uint16_t* U, int32_t r,
                            float s, uint16_t* dX, uint16_t* dA, uint16_t* dB,
                            void* ws, size_t ws_bytes, hipStream_t stream,
                            hipEvent_t ev_begin, hipEvent_t ev_end);

/* qlora_linear_fwd_noalloc -- for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): qlora_linear_fwd with the same arguments except the
 * workspace, and the same result bit for bit.  Its scratch (U and the fp32
 * partial sums) is a fixed device array of QLORA_NOALLOC_SCRATCH_BYTES that
 * the library holds on every device it runs on until the process ends; the
 * call allocates nothing (no hipMalloc, hipFree or allocating library
 * routine).  Sizes whose workspace (qlora_workspace_size(M, N, K, r, 0))
 * exceeds the array give QLORA_ERR_WORKSPACE before any launch.  Every call
 * on one device shares that device's array and leaves its contents behind;
 * calls that overlap on one device (two host threads, or two streams not
 * ordered by events) race on it and give undefined results.  The caller
 * still owns X, A, B, Y and U_out. */
#define QLORA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int32_t qlora_linear_fwd_noalloc(const nf4_tensor_t* w, const uint16_t* X,
                                 int64_t M, const uint16_t* A,
                                 const uint16_t* B, int32_t r, float s,
                                 uint16_t* Y, uint16_t* U_out,
                                 hipStream_t stream);

/* Measurement helper (not part of the layer): a read-only stream over
 * `bytes` bytes of device memory at src (16-byte aligned, bytes a multiple
 * of 16), the HBM read ceiling the few-token forward's weight stream is
 * compared with.  Every 16-byte word is read once; each of the
 * QLORA_STREAM_GRID workgroups writes one uint32 to sink[0 ..
 * QLORA_STREAM_GRID - 1] (a device buffer the caller owns).  Errors as for
 * the other calls; nothing is allocated. */
#define QLORA_STREAM_GRID 1024
int32_t qlora_stream_read(const void* src, size_t bytes, uint32_t* sink,
                          hipStream_t stream);

/* ---- Low-rank plus quantized decomposition (adapter initialization) ----
 *
 * qlora_lq_init -- split a frozen weight into a quantized part Q and a
 * rank-r part L1 L2 ("LQ-LoRA: Low-rank Plus Quantized Matrix Decomposition
 * for Efficient Language Model Finetuning", abstract: an iterative
 * algorithm; the quantized part stays fixed, the low-rank part is the
 * trained adapter).  Alternating minimization of ||W - Q - L1 L2||_F:
 *   L step: L1 L2 = rank-r approximation of W - Q, by randomized subspace
 *           iteration from the caller's Gaussian test matrix `omega`
 *           (power_iters rounds, each re-orthonormalized) and
 *           Rayleigh-Ritz on its l-dimensional range;
 *   Q step: Q = qlora_quantize(W - L1 L2) with `code_type`.
 * `start` = QLORA_LQ_START_SVD begins with Q = 0 (the first L step fits W
 * itself); QLORA_LQ_START_QUANTIZE begins with L = 0 (the first Q step is
 * plain quantization).  One iteration is one L step and one Q step.
 *
 *   W       [N, K] fp32, device; K % 64 == 0
 *   r, l    rank and subspace width: 1 <= r < l <= QLORA_LQ_MAX_L,
 *           l % 16 == 0 (l - r extra directions improve the fit)
 *   omega   [K, l] fp32, i.i.d. N(0, 1) drawn by the caller
 *   iters   1..64;  power_iters 0..16
 *   s       LoRA scale of the adapter outputs (nonzero)
 *   codes, q8, step   out: Q, as qlora_quantize writes it
 *   L1      [N, r] fp32 out;  L2t [K, r] fp32 out (L2 transposed);
 *           L1 L2t^T is the low-rank part, the factors sharing each
 *           singular value evenly (both carry its square root)
 *   A       [r, K] bf16 out = bf16(L2);  B [N, r] bf16 out = bf16(L1 / s),
 *           so that s B A ~ L1 L2 as the adapter of qlora_linear_fwd
 *   ws      device workspace, 256-byte aligned, ws_bytes >=
 *           qlora_lq_workspace_size(N, K, r, l) (about 4 N K bytes)
 * The pair returned is the last Q step's Q with the L step before it
 * (start SVD) or after it (start QUANTIZE).  Sums have a fixed order:
 * results are reproducible.  Every call raises the dynamic LDS limit of the
 * two one-workgroup solver kernels (idempotent). */
#define QLORA_LQ_MAX_L 96
#define QLORA_LQ_START_SVD 0
#define QLORA_LQ_START_QUANTIZE 1
size_t qlora_lq_workspace_size(int64_t N, int64_t K, int32_t r, int32_t l);
int32_t qlora_lq_init(const float* W, int64_t N, int64_t K, int32_t code_type,
                      int32_t r, int32_t l, const float* omega, int32_t iters,
                      int32_t power_iters, int32_t start, float s,
                      uint8_t* codes, uint8_t* q8, float* step, uint16_t* A,
                      uint16_t* B, float* L1, float* L2t, void* ws,
                      size_t ws_bytes, hipStream_t stream);

/* ---- Quantization configuration per matrix under a memory budget ----
 *
 * The LQ-LoRA abstract ("LQ-LoRA: Low-rank Plus Quantized Matrix
 * Decomposition for Efficient Language Model Finetuning") chooses each
 * matrix's quantization parameters by an integer linear program so that the
 * model meets an overall memory budget.  Here a configuration is a code type
 * (QLORA_CODE_*) and a block size (64, 128 or 256, with double
 * quantization; the layer takes all of them), its memory the state bytes
 * (qlora_config_bytes) and its error on a matrix the squared Frobenius
 * error of the quantized part.
 *
 * qlora_quant_error -- *sq_err = ||R - W_hat(R)||_F^2 in fp64, where
 * R = W, or R = W - L1 L2t^T when L1 and L2t are given (the decomposition
 * error of an LQ-LoRA initialization with that configuration), and W_hat(R)
 * is R quantized with `code_type` and dequantized (as nf4_dequantize).
 *   W      [N, K] fp32, device; K % 64 == 0
 *   L1     [N, r] fp32, L2t [K, r] fp32, device, both NULL or both given;
 *          1 <= r <= QLORA_LQ_MAX_L
 *   sq_err one double, device (8-byte aligned), written on the stream
 *   ws     device workspace, 256-byte aligned, ws_bytes >=
 *          qlora_quant_error_workspace_size(N, K, code_type, L1 != NULL)
 * The sum has a fixed order: the result is reproducible. */
size_t qlora_quant_error_workspace_size(int64_t N, int64_t K, int32_t code_type,
                                        int32_t with_lowrank);
int32_t qlora_quant_error(const float* W, int64_t N, int64_t K,
                          int32_t code_type, const float* L1, const float* L2t,
                          int32_t r, double* sq_err, void* ws, size_t ws_bytes,
                          hipStream_t stream);

/* qlora_config_error -- qlora_quant_error for any configuration: code type
 * and block size (64, 128 or 256, dividing K; the abstract's "bit-width,
 * block size"); qlora_quant_error is this call at block size 64.  The
 * workspace is sized by qlora_config_error_workspace_size. */
size_t qlora_config_error_workspace_size(int64_t N, int64_t K,
                                         int32_t code_type, int32_t blocksize,
                                         int32_t with_lowrank);
int32_t qlora_config_error(const float* W, int64_t N, int64_t K,
                           int32_t code_type, int32_t blocksize,
                           const float* L1, const float* L2t, int32_t r,
                           double* sq_err, void* ws, size_t ws_bytes,
                           hipStream_t stream);

/* qlora_ilp_plan -- host only, no device work.  Given, for M matrices and
 * C configurations, the errors err[m*C + c] (finite) and the bytes
 * bytes[m*C + c] (>= 0) (host arrays), choose one configuration per matrix
 * minimizing the total error subject to total bytes <= budget.  Solved
 * exactly (dynamic programming over the Pareto front of partial choices);
 * errors are summed in matrix order, and ties go to fewer total bytes, then
 * to the lexicographically smallest choice vector.  Writes choice[M] (host),
 * *total_err and *total_bytes; returns QLORA_ERR_INFEASIBLE if no choice
 * fits.  1 <= C <= 64. */
int32_t qlora_ilp_plan(int32_t n_matrices, int32_t n_configs, const double* err,
                       const int64_t* bytes, int64_t budget, int32_t* choice,
                       double* total_err, int64_t* total_bytes);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_NF4_H_ */
