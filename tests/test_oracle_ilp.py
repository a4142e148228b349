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


@pytest.mark.parametrize("code,bs", ilp.CONFIGS)
def test_quant_error_scales_exactly_with_powers_of_two(code, bs):
    W = (rng_for(22, 0).standard_normal((16, 256)) * 0.02).astype(np.float32)
    e = ilp.quant_error(W, code, bs)
    assert ilp.quant_error(W * np.float32(4.0), code, bs) == e * 16.0
    assert ilp.quant_error(W * np.float32(0.5), code, bs) == e / 4.0
    assert ilp.quant_error(np.zeros_like(W), code, bs) == 0.0


def test_more_bits_less_error():
    W = (rng_for(23, 0).standard_normal((64, 1024)) * 0.02).astype(np.float32)
    e = {c: ilp.quant_error(W, c) for c in ilp.CODES}
    assert e["nf4"] < e["nf3"] < e["nf2"]
    assert e["nf4"] < e["fp4"]     # NF4 fits normal weights better (blog's ablation)
    b = {c: ilp.state_bytes(64, 1024, c) for c in ilp.CODES}
    assert b["nf4"] == b["fp4"] > b["nf3"] > b["nf2"]


@pytest.mark.parametrize("bs", ilp.BLOCKSIZES)
def test_state_bytes_closed_form_by_block_size(bs):
    # codes k N K / 8, one 8-bit constant per block, one fp32 step per 256 blocks
    for N, K in [(1, 256), (3, 1024), (22016, 8192), (5120, 13824)]:
        nb = N * K // bs
        for code, k in (("nf4", 4), ("fp4", 4), ("nf3", 3), ("nf2", 2)):
            assert ilp.state_bytes(N, K, code, bs) == k * N * K // 8 + nb + 4 * (-(-nb // 256))


@pytest.mark.parametrize("code", ilp.CODES)
@pytest.mark.parametrize("bs", [128, 256])
def test_block_sizes_match_the_scalar_quantizer(code, bs):
    """The vectorized oracle at block sizes 128 and 256 against the
    element-by-element pure-Python quantizer and dequantizer (one absmax per
    `bs` elements, nearest value with ties low, 8-bit constants in groups of
    256 blocks, packing in 64-element units): bit for bit, on a weight with
    two DQ groups (the second partial), zero and tied blocks."""
    from oracle import scalar
    rows, K = (3, 22016) if bs == 256 else (3, 512)         # 256: 3 x 86 = 258 blocks
    W = (rng_for(31, bs).standard_normal((rows, K)) * 0.02).astype(np.float32)
    W[1, :bs] = 0.0                                          # an all-zero block
    W[2, bs:2 * bs] = np.float32(0.25) * nf4.code_values(code)[np.arange(bs) % nf4.code_values(code).size]
    if bs == 128:
        W = np.concatenate([W] * 44, axis=0)[:130]           # 130 x 512 / 128 = 520 blocks
    levels = [float(v) for v in nf4.code_values(code)]
    pc, pq, ps = nf4.quantize(W, blocksize=bs, code=code)
    sc, sq, ss = scalar.quantize(W.tolist(), levels, blocksize=bs)
    assert bytes(sc) == pc.tobytes()
    assert list(sq) == pq.tolist()
    assert [scalar.f32_bits(v) for v in ss] == ps.view(np.uint32).tolist()
    deq = nf4.dequantize(pc, pq, ps, *W.shape, blocksize=bs, code=code)
    assert list(scalar.dequantize(sc, sq, ss, levels, blocksize=bs)) == deq.reshape(-1).tolist()


@pytest.mark.parametrize("code", ilp.CODES)
def test_block_of_128_with_equal_half_maxima_is_two_blocks_of_64(code):
    """When both 64-element halves of every 128-element block have the same
    absmax and all blocks sit in one DQ group either way, block size 128
    gives the codes, steps and dequantized weight of block size 64, with
    each 8-bit constant repeated for the two halves."""
    rng = rng_for(32, 0)
    W = (rng.standard_normal((4, 1024)) * 0.02).astype(np.float32)   # 64 blocks of 64
    halves = W.reshape(-1, 2, 64)
    m = np.max(np.abs(halves), axis=2).max(axis=1)
    halves[:, 1, 0] = np.copysign(m, halves[:, 1, 0])   # both halves reach the pair's max
    halves[:, 0, 0] = np.copysign(m, halves[:, 0, 0])
    W = halves.reshape(4, 1024)
    c64, q64, s64 = nf4.quantize(W, blocksize=64, code=code)
    c128, q128, s128 = nf4.quantize(W, blocksize=128, code=code)
    assert np.array_equal(c64, c128)
    assert np.array_equal(s64.view(np.uint32), s128.view(np.uint32))
    assert np.array_equal(q64[0::2], q128) and np.array_equal(q64[1::2], q128)
    assert np.array_equal(nf4.dequantize(c64, q64, s64, 4, 1024, code=code),
                          nf4.dequantize(c128, q128, s128, 4, 1024, blocksize=128, code=code))


def test_error_with_low_rank_part_is_the_decomposition_objective():
    inp = draw_lq_inputs(96, 256, 8, 16, seed=24)
    state, L1, L2t = lq.decompose(inp.W, inp.Omega, 8, 1, 2)
    R = ilp.residual(inp.W, L1, L2t)
    e = ilp.quant_error(R, "nf4")
    obj = lq.objective(inp.W, nf4.quantize(R), L1, L2t)
    assert abs(np.sqrt(e) - obj) <= 1e-6 * obj
