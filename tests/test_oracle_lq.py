"""Pins for the low-rank plus quantized decomposition oracle (CPU only).

The L step is pinned to numpy's full SVD (exact on matrices of rank <= r,
and the Eckart-Young optimum when the spectrum has a gap), the Q step to the
block quantizer's own output, and the decomposition to the properties it is
built for: one quantize-first iteration is plain QLoRA plus the best fit of
its error, and the decomposition beats plain quantization on a weight with
dominant directions.
"""

import numpy as np
import pytest

from oracle import lq, nf4
from workloads import draw_lq_inputs, rng_for


def _svd_r(E, r):
    U, S, Vt = np.linalg.svd(np.asarray(E, np.float64), full_matrices=False)
    return (U[:, :r] * S[:r]) @ Vt[:r]


def test_orth_is_orthonormal_with_the_same_span():
    rng = rng_for(1, 0)
    Y = rng.standard_normal((300, 24)) @ np.diag(np.logspace(0, 3, 24))
    Q = lq.orth(Y)
    np.testing.assert_allclose(Q.T @ Q, np.eye(24), atol=1e-10)
    np.testing.assert_allclose(Q @ (Q.T @ Y), Y, rtol=0, atol=1e-9 * np.abs(Y).max())


def test_orth_drops_dependent_directions():
    rng = rng_for(1, 1)
    Y = rng.standard_normal((200, 6))
    Y = np.concatenate([Y, Y[:, :2] * 3.0], axis=1)     # rank 6 of 8 columns
    Q = lq.orth(Y)
    nz = np.linalg.norm(Q, axis=0) > 0.5
    assert nz.sum() == 6
    np.testing.assert_allclose(Q[:, nz].T @ Q[:, nz], np.eye(6), atol=1e-8)


def test_low_rank_is_exact_on_rank_r_matrices():
    rng = rng_for(2, 0)
    N, K, r, l = 160, 192, 8, 16
    E = rng.standard_normal((N, 5)) @ rng.standard_normal((5, K))     # rank 5 <= r
    L1, L2t = lq.low_rank(E, rng.standard_normal((K, l)), r, power_iters=0)
    np.testing.assert_allclose(L1 @ L2t.T, E, rtol=0, atol=1e-10 * np.abs(E).max())


def test_low_rank_reaches_the_truncated_svd_with_a_gap():
    rng = rng_for(2, 1)
    N, K, r, l = 300, 256, 10, 24
    E = (rng.standard_normal((N, r)) @ rng.standard_normal((r, K))) * 2.0 + rng.standard_normal((N, K)) * 0.1
    ref = _svd_r(E, r)
    L1, L2t = lq.low_rank(E, rng.standard_normal((K, l)), r, power_iters=2)
    assert np.linalg.norm(L1 @ L2t.T - ref) <= 1e-8 * np.linalg.norm(ref)


def test_factors_share_the_singular_values():
    rng = rng_for(2, 2)
    E = rng.standard_normal((120, 128))
    L1, L2t = lq.low_rank(E, rng.standard_normal((128, 16)), 6, power_iters=1)
    # column norms of L1 and of L2t are both sqrt(sigma_i), descending
    a, b = np.linalg.norm(L1, axis=0), np.linalg.norm(L2t, axis=0)
    np.testing.assert_allclose(a, b, rtol=1e-10)
    assert np.all(np.diff(a) <= 1e-12)
    np.testing.assert_allclose(L1.T @ L1, np.diag(a ** 2), atol=1e-10 * a.max() ** 2)


def test_quantize_first_iteration_is_plain_qlora_plus_fitted_error():
    inp = draw_lq_inputs(96, 256, 8, 16, seed=3)
    state, L1, L2t = lq.decompose(inp.W, inp.Omega, 8, iters=1, power_iters=2, start="quantize")
    plain = nf4.quantize(inp.W)
    for a, b in zip(state, plain):
        assert np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8))
    E = lq.quant_error_f32(inp.W, plain, "nf4")
    # the quantization error is nearly white: the randomized fit is close to,
    # and never better than, the optimum
    opt = np.linalg.norm(E.astype(np.float64) - _svd_r(E, 8))
    got = np.linalg.norm(E.astype(np.float64) - L1 @ L2t.T)
    assert opt <= got <= 1.02 * opt


def test_svd_first_iteration_fits_w_then_quantizes_the_rest():
    inp = draw_lq_inputs(128, 256, 8, 16, seed=4)
    ref = _svd_r(inp.W, 8)
    # the planted directions stand about 3x above the rest of the spectrum:
    # subspace iteration converges like 3^-(2 q + 1)
    for q, tol in ((2, 1e-2), (8, 1e-6)):
        state, L1, L2t = lq.decompose(inp.W, inp.Omega, 8, iters=1, power_iters=q, start="svd")
        assert np.linalg.norm(L1 @ L2t.T - ref) <= tol * np.linalg.norm(ref), q
    again = nf4.quantize(lq.residual_f32(inp.W, L1, L2t))
    for a, b in zip(state, again):
        assert np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8))


@pytest.mark.parametrize("code", ["nf4", "nf3"])
def test_decomposition_beats_plain_quantization_on_dominant_directions(code):
    inp = draw_lq_inputs(192, 512, 8, 16, seed=5)
    plain = nf4.quantize(inp.W, code=code)
    zero = np.zeros((192, 8)), np.zeros((512, 8))
    base = lq.objective(inp.W, plain, *zero, code=code)
    objs = []
    for it in (1, 2, 3):
        st, L1, L2t = lq.decompose(inp.W, inp.Omega, 8, iters=it, power_iters=2, code=code)
        objs.append(lq.objective(inp.W, st, L1, L2t, code=code))
    assert objs[0] < 0.8 * base
    assert objs[2] <= objs[0] * 1.01


def test_as_lora_reproduces_the_low_rank_term():
    rng = rng_for(6, 0)
    L1, L2t = rng.standard_normal((40, 4)), rng.standard_normal((64, 4))
    A, B = lq.as_lora(L1, L2t, 0.25)
    np.testing.assert_allclose(0.25 * B @ A, L1 @ L2t.T, rtol=1e-14)
