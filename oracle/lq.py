"""Low-rank plus quantized decomposition of a weight (oracle, numpy fp64).
Test infrastructure only.

"LQ-LoRA: Low-rank Plus Quantized Matrix Decomposition for Efficient
Language Model Finetuning", abstract: each weight is written, by an
iteration, as a quantized part plus a low-rank part held in high precision;
finetuning then trains the low-rank part and leaves the quantized part
frozen.

The abstract gives no steps.  Readings taken (listed in the design notes):

* The iteration is alternating minimization of ||W - Q - L1 L2||_F over the
  two components.  The L step takes the best rank-r approximation of
  W - Q; the Q step quantizes W - L with the block quantizer of
  :mod:`oracle.nf4` (its output is the nearest representable matrix block
  by block, not globally, so the objective need not fall at every step).
* Start: Q = 0, so the first L step is the rank-r approximation of W itself
  (``start="svd"``); or L = 0, so the first Q step is plain quantization and
  one iteration is plain QLoRA plus an adapter fitted to its error
  (``start="quantize"``).  An iteration is one L step and one Q step.
* The rank-r approximation is computed by randomized subspace iteration
  (Halko, Martinsson and Tropp, "Finding structure with randomness", 2011,
  algorithm 4.4) from a given Gaussian test matrix Omega [K, l], l > r,
  followed by the Rayleigh-Ritz step on the l-dimensional subspace (their
  algorithm 5.1 in its Gram-matrix form).
* Orthonormalization of a tall Y: Y V diag(lambda^{-1/2}) with
  Y^T Y = V diag(lambda) V^T; directions with lambda <= 1e-10 lambda_max
  are dropped (their columns set to 0).
* The two factors share the singular values evenly: L1 = Y U_r diag(lambda_r^{1/4}),
  L2^T = Z U_r diag(lambda_r^{-1/4}), where Z = E^T Y, Z^T Z = U diag(lambda) U^T
  with lambda descending, so L1 L2 = Y U_r U_r^T Y^T E.
* As a LoRA pair of scale s: A = L2 [r, K] and B = L1 / s [N, r], both
  rounded to bf16 (the adapter precision of the layer).
"""

import numpy as np

from . import nf4

DROP = 1e-10


def orth(Y: np.ndarray) -> np.ndarray:
    """Orthonormal basis of span(Y) through the Gram matrix (see module
    docstring); dropped directions give zero columns."""
    Y = np.asarray(Y, dtype=np.float64)
    lam, V = np.linalg.eigh(Y.T @ Y)
    keep = lam > DROP * lam.max()
    scale = np.zeros_like(lam)
    scale[keep] = 1.0 / np.sqrt(lam[keep])
    return Y @ (V * scale[None, :])


def range_finder(E: np.ndarray, Omega: np.ndarray, power_iters: int) -> np.ndarray:
    """Orthonormal Y [N, l] approximating the dominant l-dimensional range of
    E [N, K]: Y = E Omega, then power_iters rounds of Z = orth(E^T orth(Y)),
    Y = E Z, and a final orth."""
    E = np.asarray(E, dtype=np.float64)
    Y = E @ np.asarray(Omega, dtype=np.float64)
    for _ in range(power_iters):
        Y = orth(Y)
        Z = orth(E.T @ Y)
        Y = E @ Z
    return orth(Y)


def ritz(E: np.ndarray, Y: np.ndarray, r: int):
    """Rank-r factors from the subspace Y: returns (L1 [N, r], L2t [K, r])
    with L1 L2t^T = Y U_r U_r^T Y^T E."""
    E = np.asarray(E, dtype=np.float64)
    Z = E.T @ Y                          # = B^T, B = Y^T E
    lam, U = np.linalg.eigh(Z.T @ Z)     # = B B^T
    order = np.argsort(-lam, kind="stable")
    lam, U = lam[order][:r], U[:, order][:, :r]
    lam = np.maximum(lam, 0.0)
    d = lam ** 0.25
    dinv = np.where(d > 0, 1.0 / np.where(d > 0, d, 1.0), 0.0)
    return Y @ (U * d[None, :]), Z @ (U * dinv[None, :])


def low_rank(E: np.ndarray, Omega: np.ndarray, r: int, power_iters: int):
    """The L step: rank-r factors of E."""
    return ritz(E, range_finder(E, Omega, power_iters), r)


def residual_f32(W: np.ndarray, L1: np.ndarray, L2t: np.ndarray) -> np.ndarray:
    """fl32(W - L1 L2^T), the input of the Q step (rounded once)."""
    return (np.asarray(W, np.float64) - L1 @ L2t.T).astype(np.float32)


def quant_error_f32(W: np.ndarray, state, code: str) -> np.ndarray:
    """fl32(W - W_hat): the weight minus the dequantized (bf16) Q, one
    fp32 rounding (the input of the L step)."""
    packed, q8, step = state
    N, K = W.shape
    what = nf4.bf16_bits_to_f32(nf4.dequantize(packed, q8, step, N, K, code=code))
    return (np.asarray(W, np.float32) - what).astype(np.float32)


def decompose(W: np.ndarray, Omega: np.ndarray, r: int, iters: int, power_iters: int,
              code: str = "nf4", start: str = "svd"):
    """Alternate L and Q steps ``iters`` times.  Returns (state, L1, L2t)
    with state = (codes, q8, step) of the last Q step and L1, L2t of the last
    L step."""
    if start not in ("svd", "quantize"):
        raise ValueError("start must be 'svd' or 'quantize'")
    W = np.asarray(W, np.float32)
    state = None
    L1 = L2t = None
    for _ in range(iters):
        if start == "svd":
            E = W if state is None else quant_error_f32(W, state, code)
            L1, L2t = low_rank(E, Omega, r, power_iters)
            state = nf4.quantize(residual_f32(W, L1, L2t), code=code)
        else:
            R = W if L1 is None else residual_f32(W, L1, L2t)
            state = nf4.quantize(R, code=code)
            L1, L2t = low_rank(quant_error_f32(W, state, code), Omega, r, power_iters)
    return state, L1, L2t


def objective(W: np.ndarray, state, L1: np.ndarray, L2t: np.ndarray, code: str = "nf4") -> float:
    """||W - W_hat(Q) - L1 L2^T||_F in fp64."""
    N, K = W.shape
    packed, q8, step = state
    what = nf4.bf16_bits_to_f32(nf4.dequantize(packed, q8, step, N, K, code=code)).astype(np.float64)
    return float(np.linalg.norm(np.asarray(W, np.float64) - what - L1 @ L2t.T))


def as_lora(L1: np.ndarray, L2t: np.ndarray, s: float):
    """(A [r, K], B [N, r]) in fp64 with s B A = L1 L2 (round to bf16 for
    the layer)."""
    return L2t.T.copy(), L1 / float(s)
