"""Pins for the FP4 side of the quantizer oracle (CPU only).

The pages name FP4 as the second 4-bit data type without giving a layout;
it is read as the E2M1 element format (1 sign, 2 exponent, 1 mantissa bit,
exponent bias 1), whose eight magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4 and 6
(OCP Microscaling Formats specification v1.0, FP4 E2M1 element type), scaled
by 1/6 so that the largest is 1.  Each check ties the oracle to something
other than its own formula: the published magnitude set, exact rational
arithmetic, the pure-Python scalar quantizer, and invariants of the encoding.
"""

import math
import struct
from fractions import Fraction

import numpy as np
import pytest

from oracle import nf4, scalar
from workloads import draw_weight, WeightSpec, rng_for

FP4 = nf4.fp4_values()

# E2M1 magnitudes of codes 0..7 as published, times 6 (see module docstring)
E2M1_MAG = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2),
            Fraction(2), Fraction(3), Fraction(4), Fraction(6)]


def _nearest_f32(q: Fraction) -> np.float32:
    """The fp32 nearest to the rational q, by exact comparison with both
    fp32 neighbours of a first guess (ties cannot occur for k/12)."""
    f = np.float32(float(q))
    best = f
    for g in (np.nextafter(f, np.float32(-np.inf)), np.nextafter(f, np.float32(np.inf))):
        if abs(Fraction(float(g)) - q) < abs(Fraction(float(best)) - q):
            best = g
    return best


def test_values_are_published_e2m1_magnitudes_over_six():
    for c in range(16):
        q = (-1 if c & 8 else 1) * E2M1_MAG[c & 7] / 6
        assert FP4[c].view(np.uint32) == _nearest_f32(q).view(np.uint32) or (q == 0 and FP4[c] == 0), c
    # the sign bit is bit 3: code 8 is -0, the others mirror codes 1..7
    assert FP4[8].view(np.uint32) == np.uint32(0x80000000)
    assert np.array_equal(FP4[9:], -FP4[1:8])


def test_values_are_a_two_bit_significand_float():
    # every nonzero magnitude times 6 is m * 2^k with m in {1, 3}: one
    # implicit and at most one explicit significand bit
    for c in range(1, 8):
        mag = float(nf4.fp4_values_f64()[c]) * 6.0
        frac, _ = math.frexp(mag)
        assert (frac * 4.0).is_integer(), (c, mag)
    # max 6, min normal 1, min subnormal 1/2 (times 1/6)
    assert float(FP4[7]) == 1.0
    assert abs(float(FP4[2]) - 1 / 6) < 1e-7 and abs(float(FP4[1]) - 1 / 12) < 1e-8


def test_fp4_is_monotone_in_the_magnitude_bits():
    pos = FP4[:8].astype(np.float64)
    assert np.all(np.diff(pos) > 0)
    assert len(set(FP4.astype(np.float64).tolist())) == 15   # +0 and -0 coincide


def _transition_points():
    """For each pair of consecutive distinct values, the two fp32 numbers
    around their exact midpoint, with the expected (lower, upper) codes."""
    dist = sorted(set(float(v) for v in FP4))
    code_of = {}
    for c in range(16):
        code_of.setdefault(float(FP4[c]), c)      # lowest code of each value
    xs, expect = [], []
    for a, b in zip(dist[:-1], dist[1:]):
        mid = Fraction(a) / 2 + Fraction(b) / 2
        f = np.float32(float(mid))
        lo = f if Fraction(float(f)) <= mid else np.nextafter(f, np.float32(-np.inf))
        hi = np.nextafter(lo, np.float32(np.inf))
        xs += [lo, hi]
        # at an exact fp32 midpoint the tie goes to the lower value
        expect += [code_of[a], code_of[b]]
    return np.array(xs, np.float32), expect


def test_nearest_code_transition_points():
    xs, expect = _transition_points()
    assert list(nf4.nearest_code(xs, FP4)) == expect
    # values map to their own code, except -0 which maps to +0 (code 0)
    own = list(nf4.nearest_code(FP4, FP4))
    assert own == [0] + list(range(1, 8)) + [0] + list(range(9, 16))
    assert nf4.nearest_code(np.array([-0.0, 0.0], np.float32), FP4).tolist() == [0, 0]


def test_exact_ties_go_to_the_lower_value():
    # the midpoint of 0 and 1/12 is fl32(1/12)/2, an fp32 number: +-x tie
    h = np.float32(FP4[1] / np.float32(2))
    assert Fraction(float(h)) * 2 == Fraction(float(FP4[1]))
    got = nf4.nearest_code(np.array([h, -h], np.float32), FP4).tolist()
    assert got == [0, 9]           # +x: 0 below 1/12; -x: -1/12 below 0


def test_nearest_code_matches_exact_bruteforce():
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.uniform(-1, 1, 3000), rng.standard_normal(500) * 0.05]).astype(np.float32)
    x = np.clip(x, -1, 1)
    got = nf4.nearest_code(x, FP4)
    vals = [Fraction(float(v)) for v in FP4]
    for xi, g in zip(x, got):
        fx = Fraction(float(xi))
        d = [abs(fx - v) for v in vals]
        m = min(d)
        cands = [c for c in range(16) if d[c] == m]
        low = min(vals[c] for c in cands)
        want = min(c for c in cands if vals[c] == low)
        assert g == want, (float(xi), g, want)


def _tiny_fp4_weights():
    rng = np.random.default_rng(3)
    cases = {
        "normal": (rng.standard_normal((2, 256)) * 0.02).astype(np.float32),
        "with_zero_block": np.concatenate(
            [np.zeros((1, 64)), rng.standard_normal((1, 64))], axis=1).astype(np.float32),
        "signed_zeros": np.array([[0.0, -0.0] * 32 + list(rng.standard_normal(64))], np.float32),
    }
    xs, _ = _transition_points()
    row = list(xs) + [1.0, -1.0]
    row += [0.0] * (64 - len(row) % 64) if len(row) % 64 else []
    cases["transition_points"] = np.array([row], np.float32)
    return cases


@pytest.mark.parametrize("name", list(_tiny_fp4_weights().keys()))
def test_fp4_quantizer_matches_scalar_bruteforce(name):
    W = _tiny_fp4_weights()[name]
    packed, q8, step = nf4.quantize(W, code="fp4")
    lv = [float(v) for v in FP4]
    sp_, sq, ss = scalar.quantize(W.tolist(), lv)
    assert bytes(packed.tobytes()) == sp_
    assert list(q8) == sq
    assert [struct.pack("<f", v) for v in step] == [struct.pack("<f", v) for v in ss]
    deq = nf4.dequantize(packed, q8, step, *W.shape, code="fp4")
    assert list(deq.reshape(-1)) == scalar.dequantize(sp_, sq, ss, lv)


def test_fp4_all_zero_weight_uses_code_zero():
    W = np.zeros((2, 128), np.float32)
    packed, q8, step = nf4.quantize(W, code="fp4")
    assert np.all(packed == 0) and np.all(q8 == 0) and np.all(step == 0)


def test_fp4_absmax_element_maps_to_an_end_code():
    W = draw_weight(WeightSpec("w", 32, 512, 0.02, heavy_frac=0.01), rng_for(5, 0))
    Wb = W.reshape(-1, 64)
    codes = nf4.unpack_codes(nf4.quantize(W, code="fp4")[0]).reshape(-1, 64)
    j = np.argmax(np.abs(Wb), axis=1)
    sel = codes[np.arange(len(j)), j]
    sgn = Wb[np.arange(len(j)), j] > 0
    assert np.all(np.where(sgn, sel == 7, sel == 15))


def test_fp4_round_trip_error_bound():
    # the widest gap between FP4 values is 2/6 (between 4/6 and 1), so the
    # code error is at most c/6; the 8-bit constant adds at most step/2
    W = draw_weight(WeightSpec("w", 64, 1024, 0.02, heavy_frac=0.01), rng_for(6, 0))
    packed, q8, step = nf4.quantize(W, code="fp4")
    what = nf4.bf16_bits_to_f32(nf4.dequantize(packed, q8, step, *W.shape, code="fp4"))
    c = nf4.block_absmax(W).astype(np.float64)
    st = step.astype(np.float64)[np.arange(c.size) // 256]
    err = np.abs(W.astype(np.float64).reshape(-1, 64) - what.astype(np.float64).reshape(-1, 64))
    bound = (1 / 6) * c + 0.5 * st
    slack = 2.0 ** -9 * np.abs(what.reshape(-1, 64)) + 1e-6 * c[:, None]
    assert np.all(err <= bound[:, None] + slack)
    # and the bound is nearly reached: FP4 is coarser than NF4 at the top
    rel = err / c[:, None]
    assert rel.max() > 0.12


def test_fp4_scaled_values_give_their_codes():
    c = np.float32(2.0 ** -4)
    row = np.tile(FP4 * c, 4).astype(np.float32)
    codes = nf4.unpack_codes(nf4.quantize(row[None, :], code="fp4")[0])
    want = [0] + list(range(1, 8)) + [0] + list(range(9, 16))
    assert list(codes) == want * 4
