"""Pins for the fp64 layer oracle (CPU only): torch autograd on the forward
definition, central finite differences, special cases and bilinear
identities."""

import numpy as np
import pytest
import torch

from oracle import linear, nf4


def _tiny(M=3, N=5, K=64, r=2, seed=0):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((M, K))
    W = rng.standard_normal((N, K)) * 0.02
    A = rng.standard_normal((r, K)) * 0.1
    B = rng.standard_normal((N, r)) * 0.1
    dY = rng.standard_normal((M, N))
    return X, W, A, B, dY


@pytest.mark.parametrize("shape", [(3, 5, 64, 2), (7, 16, 128, 8), (1, 9, 64, 1)])
def test_backward_matches_torch_autograd(shape):
    M, N, K, r = shape
    X, W, A, B, dY = _tiny(M, N, K, r, seed=M + N)
    s = 0.75
    tX = torch.tensor(X, requires_grad=True)
    tA = torch.tensor(A, requires_grad=True)
    tB = torch.tensor(B, requires_grad=True)
    tW = torch.tensor(W)
    Y = tX @ tW.T + s * (tX @ tA.T) @ tB.T
    Y.backward(torch.tensor(dY))
    np.testing.assert_allclose(linear.forward(X, W, A, B, s), Y.detach().numpy(), rtol=1e-13, atol=1e-14)
    dX, dA, dB = linear.backward(X, dY, W, A, B, s)
    np.testing.assert_allclose(dX, tX.grad.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dA, tA.grad.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dB, tB.grad.numpy(), rtol=1e-12, atol=1e-13)
    gA, gB = linear.adapter_grads(X, dY, A, B, s)
    np.testing.assert_allclose(gA, tA.grad.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(gB, tB.grad.numpy(), rtol=1e-12, atol=1e-13)


def test_backward_matches_finite_differences():
    X, W, A, B, dY = _tiny()
    s = 2.0

    def loss(X_, A_, B_):
        return float(np.sum(dY * linear.forward(X_, W, A_, B_, s)))

    dX, dA, dB = linear.backward(X, dY, W, A, B, s)
    h = 1e-5
    for arr, grad, name in ((X, dX, "X"), (A, dA, "A"), (B, dB, "B")):
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            p = arr.copy(); p[idx] += h
            m = arr.copy(); m[idx] -= h
            args = {"X": (X, A, B), "A": (X, A, B), "B": (X, A, B)}[name]
            ap = list(args); am = list(args)
            pos = "XAB".index(name)
            ap[pos] = p; am[pos] = m
            fd[idx] = (loss(*ap) - loss(*am)) / (2 * h)
        np.testing.assert_allclose(grad, fd, rtol=1e-7, atol=1e-9, err_msg=name)


def test_identity_input_returns_transposed_weight():
    K, N, r = 64, 8, 4
    rng = np.random.default_rng(1)
    W = rng.standard_normal((N, K))
    A = rng.standard_normal((r, K))
    B = np.zeros((N, r))
    Y = linear.forward(np.eye(K), W, A, B, 3.0)
    assert np.array_equal(Y, W.T)


def test_zero_weight_isolates_lora():
    X, W, A, B, dY = _tiny(4, 6, 64, 3)
    s = 0.5
    Z = np.zeros_like(W)
    Y = linear.forward(X, Z, A, B, s)
    np.testing.assert_allclose(Y, s * (X @ A.T) @ B.T, rtol=1e-14)
    dX, _, _ = linear.backward(X, dY, Z, A, B, s)
    np.testing.assert_allclose(dX, (s * dY @ B) @ A, rtol=1e-13)


def test_zero_adapter_is_plain_matmul():
    X, W, A, B, dY = _tiny(4, 6, 64, 3)
    ref = torch.tensor(X) @ torch.tensor(W).T
    np.testing.assert_allclose(linear.forward(X, W, A, np.zeros_like(B), 1.0), ref.numpy(), rtol=1e-14)
    np.testing.assert_allclose(linear.forward(X, W, np.zeros_like(A), B, 1.0), ref.numpy(), rtol=1e-14)
    dX, dA, dB = linear.backward(X, dY, W, np.zeros_like(A), B, 1.0)
    assert np.all(dB == 0)


def test_bilinear_identities():
    X, W, A, B, dY = _tiny(6, 10, 128, 4, seed=9)
    s = 1.25
    Y = linear.forward(X, W, A, B, s)
    Yb = linear.forward_base(X, W)
    dX, dA, dB = linear.backward(X, dY, W, A, B, s)
    # Y is linear in X, and of degree one in A and in B
    np.testing.assert_allclose(np.sum(dY * Y), np.sum(dX * X), rtol=1e-12)
    np.testing.assert_allclose(np.sum(dA * A), np.sum(dY * (Y - Yb)), rtol=1e-12)
    np.testing.assert_allclose(np.sum(dB * B), np.sum(dY * (Y - Yb)), rtol=1e-12)


def test_row_sampled_helpers_match_full():
    X, W, A, B, dY = _tiny(9, 7, 64, 2, seed=4)
    rows = [0, 3, 8]
    np.testing.assert_allclose(linear.forward_rows(X, W, A, B, 0.3, rows),
                               linear.forward(X, W, A, B, 0.3)[rows], rtol=1e-14)
    np.testing.assert_allclose(linear.backward_rows(X, dY, W, A, B, 0.3, rows),
                               linear.backward(X, dY, W, A, B, 0.3)[0][rows], rtol=1e-14)


def test_forward_on_dequantized_weight_tracks_fp32_weight():
    # The frozen NF4 base changes Y by at most the round-trip error bound.
    rng = np.random.default_rng(2)
    W = (rng.standard_normal((32, 256)) * 0.02).astype(np.float32)
    packed, q8, step = nf4.quantize(W)
    what = nf4.bf16_bits_to_f32(nf4.dequantize(packed, q8, step, 32, 256))
    X = rng.standard_normal((4, 256))
    d = linear.forward_base(X, what) - linear.forward_base(X, W)
    c = nf4.block_absmax(W).reshape(32, 4)
    bound = np.abs(X) @ np.repeat(0.16 * c + 0.5 * step[0], 64, axis=1).T
    assert np.all(np.abs(d) <= bound)
