"""Per-matrix choice of quantization configuration under a memory budget
(oracle).  Test infrastructure only.

"LQ-LoRA: Low-rank Plus Quantized Matrix Decomposition for Efficient
Language Model Finetuning", abstract: an integer linear program picks the
quantization parameters (for example bit width and block size) of each
matrix so that the model meets an overall memory budget.

Readings taken (listed in the design notes):

* A configuration is a code type of the block quantizer (NF4, FP4, NF3,
  NF2) and a block size (64, 128 or 256 consecutive elements of the
  row-major weight share one absmax constant), with the constants double
  quantized in groups of 256 blocks as at block size 64; the codes are
  packed in 64-element units whatever the block size.  Its memory is the
  bytes of the stored state (codes + 8-bit constants + fp32 steps).
* The error of matrix m under configuration c is the squared Frobenius
  error of its quantized part: ||R - W_hat_c(R)||_F^2 with R = W (plain
  QLoRA) or R = fl32(W - L1 L2^T) when a low-rank part is given (then it is
  the decomposition error ||W - L - Q||^2 up to the rounding of R).
* The program: choose one configuration per matrix, minimize the total
  error, subject to total bytes <= budget.  It is solved exactly; ties go
  to the smaller total bytes, then to the lexicographically smallest choice
  vector.  The oracle enumerates every assignment (small instances only).
"""

import itertools

import numpy as np

from . import nf4

CODES = ("nf4", "fp4", "nf3", "nf2")
BLOCKSIZES = (64, 128, 256)
# every (code type, block size) pair, code type major
CONFIGS = tuple((c, b) for c in CODES for b in BLOCKSIZES)


def residual(W, L1=None, L2t=None) -> np.ndarray:
    if L1 is None:
        return np.asarray(W, np.float32)
    return (np.asarray(W, np.float64) - np.asarray(L1, np.float64) @ np.asarray(L2t, np.float64).T
            ).astype(np.float32)


def quant_error(R, code: str, blocksize: int = nf4.BLOCKSIZE) -> float:
    """||R - W_hat(R)||_F^2 in fp64 for one configuration."""
    R = np.asarray(R, np.float32)
    N, K = R.shape
    packed, q8, step = nf4.quantize(R, blocksize=blocksize, code=code)
    what = nf4.bf16_bits_to_f32(nf4.dequantize(packed, q8, step, N, K, blocksize=blocksize,
                                               code=code))
    d = R.astype(np.float64) - what.astype(np.float64)
    return float(np.sum(d * d))


def state_bytes(N: int, K: int, code: str, blocksize: int = nf4.BLOCKSIZE) -> int:
    return nf4.storage_bytes(N, K, blocksize=blocksize, code=code)


def plan(err, nbytes, budget: int):
    """Exact solution by enumeration.  err, nbytes: [M][C].  Returns
    (choice tuple, total error, total bytes), or None if nothing fits."""
    err = np.asarray(err, np.float64)
    nbytes = np.asarray(nbytes, np.int64)
    M, C = err.shape
    best = None
    for choice in itertools.product(range(C), repeat=M):
        b = 0
        e = 0.0
        for m, c in enumerate(choice):   # sums in matrix order
            b += int(nbytes[m, c])
            e += float(err[m, c])
        if b > budget:
            continue
        key = (e, b, choice)
        if best is None or key < best:
            best = key
    if best is None:
        return None
    e, b, choice = best
    return choice, e, b
