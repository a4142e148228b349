"""Pins for the per-matrix configuration program (oracle.ilp; CPU only):
a hand-solved instance, the unconstrained and tightest budgets, exact
power-of-two scaling of the quantization error, its order across bit
widths, and agreement with the decomposition objective."""

import numpy as np
import pytest

from oracle import ilp, lq, nf4
from workloads import draw_lq_inputs, rng_for


def test_hand_solved_instance():
    # Three matrices, two configurations (0: 20 bytes, accurate; 1: 10 bytes,
    # coarse).  Upgrading matrix m from 1 to 0 costs 10 bytes and saves
    # s = (5, 9, 2) error.  Budget 50 = 30 + 20 allows two upgrades: the two
    # largest savings are matrices 1 and 0, so the choice is (0, 0, 1) with
    # error 1 + 2 + 5 = 8.  Budget 49 allows one upgrade (matrix 1); budget
    # 29 is below the 30 bytes of the smallest configurations.
    err = [[1.0, 6.0], [2.0, 11.0], [3.0, 5.0]]
    nbytes = [[20, 10], [20, 10], [20, 10]]
    choice, e, b = ilp.plan(err, nbytes, 50)
    assert choice == (0, 0, 1) and e == 8.0 and b == 50
    # one upgrade only: matrix 1 (largest saving)
    assert ilp.plan(err, nbytes, 49)[0] == (1, 0, 1)
    assert ilp.plan(err, nbytes, 29) is None


def test_unconstrained_and_tightest_budgets():
    rng = rng_for(21, 0)
    err = rng.random((5, 4))
    nbytes = rng.integers(10, 100, (5, 4))
    choice, _, _ = ilp.plan(err, nbytes, 10 ** 9)
    assert list(choice) == list(np.argmin(err, axis=1))
    tight = int(np.sum(np.min(nbytes, axis=1)))
    choice, _, b = ilp.plan(err, nbytes, tight)
    assert b == tight
    assert all(nbytes[m][c] == np.min(nbytes[m]) for m, c in enumerate(choice))


def test_ties_go_to_fewer_bytes_then_smaller_choice():
    err = [[1.0, 1.0], [2.0, 2.0]]
    nbytes = [[10, 5], [7, 7]]
    assert ilp.plan(err, nbytes, 100)[0] == (1, 0)


@pytest.mark.parametrize("code", ilp.CONFIGS)
def test_quant_error_scales_exactly_with_powers_of_two(code):
    W = (rng_for(22, 0).standard_normal((16, 256)) * 0.02).astype(np.float32)
    e = ilp.quant_error(W, code)
    assert ilp.quant_error(W * np.float32(4.0), code) == e * 16.0
    assert ilp.quant_error(W * np.float32(0.5), code) == e / 4.0
    assert ilp.quant_error(np.zeros_like(W), code) == 0.0


def test_more_bits_less_error():
    W = (rng_for(23, 0).standard_normal((64, 1024)) * 0.02).astype(np.float32)
    e = {c: ilp.quant_error(W, c) for c in ilp.CONFIGS}
    assert e["nf4"] < e["nf3"] < e["nf2"]
    assert e["nf4"] < e["fp4"]     # NF4 fits normal weights better (blog's ablation)
    b = {c: ilp.state_bytes(64, 1024, c) for c in ilp.CONFIGS}
    assert b["nf4"] == b["fp4"] > b["nf3"] > b["nf2"]


def test_error_with_low_rank_part_is_the_decomposition_objective():
    inp = draw_lq_inputs(96, 256, 8, 16, seed=24)
    state, L1, L2t = lq.decompose(inp.W, inp.Omega, 8, 1, 2)
    R = ilp.residual(inp.W, L1, L2t)
    e = ilp.quant_error(R, "nf4")
    obj = lq.objective(inp.W, nf4.quantize(R), L1, L2t)
    assert abs(np.sqrt(e) - obj) <= 1e-6 * obj
