"""The frozen-NF4-base + LoRA linear layer in fp64.  Test infrastructure only.

Shapes follow the torch Linear convention: X [M, K], W [N, K], A [r, K],
B [N, r], Y [M, N]; s = alpha / r.

* The base weight is stored in 4 bits and dequantized to 16 bits for every
  forward and backward pass; the base never changes and only the adapters
  receive gradients ("QLoRA: fine-tuning a 65B model on one GPU", section
  "Where the memory goes"; "QLoRA: efficient finetuning of quantized LLMs",
  Abstract: gradients are backpropagated through the frozen 4-bit model
  into the low-rank adapters).
* LoRA trains a low-rank pair beside the frozen weight (blog, same section).
  With the adapter written as the product B A scaled by s, the forward pass
  is Y = X W_hat^T + s (X A^T) B^T.
* The backward pass re-materializes the low-precision weight rather than
  keeping a 16-bit copy ("ModuLoRA: ...", abstract).  Mathematically it is
  the chain rule of the forward pass: with U = X A^T and dU = s dY B,
  dX = dY W_hat + dU A, dA = dU^T X, dB = s dY^T U, and no gradient for W.

All products are fp64 numpy matmuls on the exact values of the bf16 inputs
and of the bit-exact dequantized weight; there is no blocking or reordering
beyond what numpy's matmul does internally.
"""

import numpy as np


def as_f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def lora_down(X, A) -> np.ndarray:
    """U = X A^T  [M, r]."""
    return as_f64(X) @ as_f64(A).T


def forward(X, W_hat, A, B, s: float) -> np.ndarray:
    """Y = X W_hat^T + s (X A^T) B^T  [M, N]."""
    X = as_f64(X)
    U = lora_down(X, A)
    return X @ as_f64(W_hat).T + float(s) * (U @ as_f64(B).T)


def forward_base(X, W_hat) -> np.ndarray:
    """The frozen part alone, X W_hat^T."""
    return as_f64(X) @ as_f64(W_hat).T


def backward(X, dY, W_hat, A, B, s: float):
    """Gradients of <dY, Y> with respect to X, A and B.

    Returns (dX [M, K], dA [r, K], dB [N, r]).  There is no dW: the base
    weight is frozen.
    """
    X = as_f64(X)
    dY = as_f64(dY)
    A = as_f64(A)
    B = as_f64(B)
    s = float(s)
    U = X @ A.T
    dU = s * (dY @ B)
    dX = dY @ as_f64(W_hat) + dU @ A
    dA = dU.T @ X
    dB = s * (dY.T @ U)
    return dX, dA, dB


def backward_rows(X, dY, W_hat, A, B, s: float, rows):
    """dX restricted to the given rows (dX row m depends only on dY row m);
    for checking large shapes on a sample of rows."""
    rows = np.asarray(rows)
    dYr = as_f64(dY)[rows]
    dU = float(s) * (dYr @ as_f64(B))
    return dYr @ as_f64(W_hat) + dU @ as_f64(A)


def forward_rows(X, W_hat, A, B, s: float, rows):
    """Y restricted to the given rows."""
    rows = np.asarray(rows)
    return forward(as_f64(X)[rows], W_hat, A, B, s)


def adapter_grads(X, dY, A, B, s: float):
    """dA and dB alone, in full, without the M x N x K product of dX
    (same chain rule as ``backward``); for checking large shapes."""
    X = as_f64(X)
    dY = as_f64(dY)
    s = float(s)
    U = X @ as_f64(A).T
    dU = s * (dY @ as_f64(B))
    return dU.T @ X, s * (dY.T @ U)
