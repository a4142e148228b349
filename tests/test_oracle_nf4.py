"""Pins for the NF4 quantizer oracle (CPU only).

Each check ties the oracle to something other than itself: scipy's normal
quantile and CDF, torch's bf16 cast, a pure-Python scalar quantizer,
closed forms and invariants of the encoding.
"""

import math
import struct

import numpy as np
import pytest
import scipy.special as sp
import torch

from oracle import nf4, scalar
from workloads import draw_weight, WeightSpec, rng_for

LEVELS = nf4.nf4_levels()
LV = LEVELS.astype(np.float64)


# ---------------------------------------------------------------- levels

def test_normal_quantile_matches_scipy():
    ps = np.concatenate([np.linspace(0.5, 0.999, 257), [nf4.NF4_DELTA]])
    for p in ps:
        ours = nf4.normal_quantile(float(p))
        ref = float(sp.ndtri(p))
        # both sides are accurate to a few ulp of p, amplified by 1/phi(x)
        cond = 2.2e-16 / (np.exp(-0.5 * ref * ref) / np.sqrt(2 * np.pi))
        assert abs(ours - ref) <= 4 * cond + 4e-15 * abs(ref), (p, ours, ref)


def test_levels_match_independent_scipy_construction():
    d = 1.0 - 0.5 * (1.0 / 30 + 1.0 / 32)
    z = sp.ndtri(d)
    pos = sp.ndtri(np.linspace(d, 0.5, 9)[:-1]) / z
    neg = -sp.ndtri(np.linspace(d, 0.5, 8)[:-1]) / z
    ref = np.sort(np.concatenate([neg, [0.0], pos]))
    ours = nf4.nf4_levels_f64()
    np.testing.assert_allclose(ours, ref, rtol=1e-14, atol=1e-15)
    assert np.array_equal(ref.astype(np.float32).view(np.uint32), LEVELS.view(np.uint32))


def test_levels_far_from_fp32_rounding_boundaries():
    # The fp32 bits cannot depend on how Phi^{-1} was computed: every level
    # lies well inside its fp32 rounding interval.
    v = nf4.nf4_levels_f64()
    for x in v:
        if x in (-1.0, 0.0, 1.0):
            continue
        f = np.float32(x)
        up = np.nextafter(f, np.float32(np.inf))
        dn = np.nextafter(f, np.float32(-np.inf))
        lo_b = (float(f) + float(dn)) / 2
        hi_b = (float(f) + float(up)) / 2
        margin = min(x - lo_b, hi_b - x) / abs(x)
        assert margin > 1e-9, (x, margin)


def test_levels_invariants():
    assert LEVELS.shape == (16,)
    assert np.all(np.diff(LV) > 0), "strictly increasing"
    assert LEVELS[0] == -1.0 and LEVELS[15] == 1.0
    assert LEVELS.view(np.uint32)[7] == 0, "exact +0"
    assert np.sum(LV < 0) == 7 and np.sum(LV > 0) == 8
    gaps = np.diff(LV)
    assert np.argmax(gaps) == 0
    assert abs(gaps.max() / 2 - 0.15190) < 1e-4


def test_levels_cover_equal_shares():
    # The probability positions behind the levels are evenly spaced on each
    # side of zero: equal probability mass between consecutive levels.
    d = nf4.NF4_DELTA
    z = sp.ndtri(d)
    p = sp.ndtr(nf4.nf4_levels_f64() * z)
    pos = p[8:]
    neg = 1.0 - p[:7]
    np.testing.assert_allclose(np.diff(pos), (d - 0.5) / 8, rtol=0, atol=1e-13)
    np.testing.assert_allclose(np.diff(neg[::-1]), (d - 0.5) / 7, rtol=0, atol=1e-13)
    np.testing.assert_allclose(pos[-1], d, atol=1e-14)
    np.testing.assert_allclose(neg[0], d, atol=1e-14)
    np.testing.assert_allclose(pos[0], 0.5 + (d - 0.5) / 8, atol=1e-14)


def test_levels_golden_fixture():
    path = __file__.replace("test_oracle_nf4.py", "golden/nf4_levels_fp32.txt")
    bits = [int(tok, 16) for line in open(path) if not line.startswith("#")
            for tok in line.split()]
    assert bits == [int(b) for b in LEVELS.view(np.uint32)]


# ---------------------------------------------------------------- nearest level

def test_nearest_level_transition_points():
    # Nearest-level coding is a monotone step function of x.  It changes
    # exactly where x passes the midpoint of two neighbouring levels; at an
    # fp32 midpoint the tie goes to the lower level.
    xs, expect = [], []
    for i in range(15):
        mid = (LV[i] + LV[i + 1]) / 2
        f = np.float32(mid)
        lo = f if float(f) <= mid else np.nextafter(f, np.float32(-np.inf))
        hi = np.nextafter(lo, np.float32(np.inf))
        xs += [lo, hi]
        expect += [i, i + 1]
    got = nf4.nearest_level(np.array(xs, dtype=np.float32), LEVELS)
    assert list(got) == expect
    # the levels themselves map to their own index, and -0.0 to the zero
    assert list(nf4.nearest_level(LEVELS, LEVELS)) == list(range(16))
    assert nf4.nearest_level(np.array([-0.0], np.float32), LEVELS)[0] == 7


def test_nearest_level_matches_scalar_on_random_fp32():
    rng = np.random.default_rng(1)
    x = rng.uniform(-1, 1, 4000).astype(np.float32)
    got = nf4.nearest_level(x, LEVELS)
    lv = [float(v) for v in LEVELS]
    for xi, g in zip(x, got):
        d = [abs(float(xi) - v) for v in lv]
        assert g == d.index(min(d))


# ---------------------------------------------------------------- bf16

def _bf16_cases():
    rng = np.random.default_rng(2)
    x = [rng.standard_normal(20000).astype(np.float32),
         (rng.standard_normal(2000) * 1e-38).astype(np.float32),   # subnormals
         np.clip(rng.standard_normal(2000) * 1.5e38, -3.4e38, 3.4e38).astype(np.float32)]
    # exact ties with even and odd kept bits, both signs
    u = rng.integers(0, 0x7F80, 2000).astype(np.uint32) << np.uint32(16)   # finite only
    u |= np.uint32(0x8000)
    u |= (rng.integers(0, 2, 2000).astype(np.uint32) << np.uint32(31))
    x.append(u.view(np.float32))
    x.append(np.array([0.0, -0.0, 1.0, -1.0, 3.3895314e38, -3.3895314e38,
                       1e-45, -1e-45], dtype=np.float32))
    return np.concatenate(x)


def test_bf16_rne_matches_torch():
    x = _bf16_cases()
    ours = nf4.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_rne_matches_scalar_neighbour_rule():
    x = _bf16_cases()[::7]
    ours = nf4.f32_to_bf16_bits(x)
    for xi, o in zip(x, ours):
        assert scalar.bf16_bits(float(xi)) == int(o), hex(struct.unpack("<I", struct.pack("<f", xi))[0])


# ---------------------------------------------------------------- quantizer vs scalar brute force

def _tiny_weights():
    rng = np.random.default_rng(3)
    cases = {
        "1x64": (rng.standard_normal((1, 64)) * 0.02).astype(np.float32),
        "2x128": (rng.standard_normal((2, 128)) * 0.02).astype(np.float32),
        "3x1024_partial_group": (rng.standard_normal((3, 1024)) * 0.02).astype(np.float32),
        "5x4096_two_groups": (rng.standard_normal((5, 4096)) * 0.02).astype(np.float32),
    }
    den = (rng.standard_normal((1, 128)) * 1e-39).astype(np.float32)
    cases["subnormal_block"] = den
    one = np.zeros((2, 64), np.float32)
    one[0, 17] = -0.3
    one[1, 5] = 1e-30
    cases["single_nonzero"] = one
    cases["zeros_and_neg_zero"] = np.array([[0.0, -0.0] * 32], np.float32)
    # ties: x exactly at an fp32-representable midpoint is rare, so build
    # blocks whose normalized values sit exactly on the transition points
    tie = []
    for i in range(15):
        mid = (LV[i] + LV[i + 1]) / 2
        f = np.float32(mid)
        lo = f if float(f) <= mid else np.nextafter(f, np.float32(-np.inf))
        tie += [lo, np.nextafter(lo, np.float32(np.inf))]
    tie += [1.0, -1.0]                                          # c = 1 exactly
    cases["transition_points"] = np.array([tie + tie[::-1]], np.float32)
    return cases


@pytest.mark.parametrize("name", list(_tiny_weights().keys()))
def test_quantizer_matches_scalar_bruteforce(name):
    W = _tiny_weights()[name]
    packed, q8, step = nf4.quantize(W)
    sp_, sq, ss = scalar.quantize(W.tolist(), [float(v) for v in LEVELS])
    assert bytes(packed.tobytes()) == sp_
    assert list(q8) == sq
    assert [struct.pack("<f", v) for v in step] == [struct.pack("<f", v) for v in ss]
    deq = nf4.dequantize(packed, q8, step, *W.shape)
    sd = scalar.dequantize(sp_, sq, ss, [float(v) for v in LEVELS])
    assert list(deq.reshape(-1)) == sd


# ---------------------------------------------------------------- invariants

def _random_heavy(N=64, K=512, seed=5):
    return draw_weight(WeightSpec("w", N, K, 0.02, heavy_frac=0.01), rng_for(seed, 0))


def test_code_is_nearest_within_half_gap():
    W = _random_heavy()
    c = nf4.block_absmax(W)
    x = nf4.normalize(W, c).astype(np.float64).reshape(-1)
    k = nf4.unpack_codes(nf4.quantize(W)[0]).astype(np.int64)
    lk = LV[k]
    above = x >= lk
    up_gap = LV[np.minimum(k + 1, 15)] - lk          # 0 for k = 15
    dn_gap = lk - LV[np.maximum(k - 1, 0)]           # 0 for k = 0
    assert np.all(np.where(above, x - lk <= up_gap / 2, lk - x <= dn_gap / 2))
    assert np.all((x <= 1.0) & (x >= -1.0))


def test_absmax_element_maps_to_an_end_code():
    W = _random_heavy()
    Wb = W.reshape(-1, 64)
    codes = nf4.unpack_codes(nf4.quantize(W)[0]).reshape(-1, 64)
    j = np.argmax(np.abs(Wb), axis=1)
    sel = codes[np.arange(len(j)), j]
    sgn = Wb[np.arange(len(j)), j] > 0
    assert np.all(np.where(sgn, sel == 15, sel == 0))


def test_round_trip_error_bound():
    W = _random_heavy(128, 1024)
    packed, q8, step = nf4.quantize(W)
    what = nf4.bf16_bits_to_f32(nf4.dequantize(packed, q8, step, *W.shape)).astype(np.float64)
    c = nf4.block_absmax(W).astype(np.float64)
    st = step.astype(np.float64)[np.arange(c.size) // 256]
    bound = 0.15190 * c + 0.5 * st
    err = np.abs(W.astype(np.float64).reshape(-1, 64) - what.reshape(-1, 64))
    slack = 2.0 ** -9 * np.abs(what.reshape(-1, 64)) + 1e-6 * c[:, None]
    assert np.all(err <= bound[:, None] + slack)


def test_code_histogram_entropy_for_normal_blocks():
    rng = np.random.default_rng(7)
    W = rng.standard_normal((256, 1024)).astype(np.float32)
    codes = nf4.unpack_codes(nf4.quantize(W)[0])
    h = np.bincount(codes, minlength=16) / codes.size
    ent = -np.sum(h[h > 0] * np.log2(h[h > 0]))
    # every level in use, spread close to evenly (4 bits would be perfect)
    assert np.all(h > 0.01) and 3.8 < ent < 3.95


# ---------------------------------------------------------------- special cases

def test_all_zero_weight():
    W = np.zeros((4, 256), np.float32)
    packed, q8, step = nf4.quantize(W)
    assert np.all(packed == 0x77) and np.all(q8 == 0) and np.all(step == 0)
    deq = nf4.dequantize(packed, q8, step, 4, 256)
    assert np.all(deq == 0)


def test_power_of_two_group_max_gives_exact_step():
    e = -7
    W = np.zeros((1, 64 * 4), np.float32)
    W[0, 0] = 255 * 2.0 ** e
    W[0, 64:128] = 0.001
    packed, q8, step = nf4.quantize(W)
    assert step[0] == np.float32(2.0 ** e)
    assert q8[0] == 255


def test_scaled_level_block_gives_codes_in_order():
    c = np.float32(2.0 ** -5)
    row = np.tile(LEVELS * c, 4).astype(np.float32)
    packed, _, _ = nf4.quantize(row[None, :])
    codes = nf4.unpack_codes(packed)
    assert list(codes) == list(range(16)) * 4


def test_nibble_order_even_element_low():
    W = np.zeros((1, 64), np.float32)
    W[0, 0] = 1.0   # code 15
    W[0, 1] = -1.0  # code 0
    W[0, 2] = -1.0  # code 0
    W[0, 3] = 1.0   # code 15
    packed, _, _ = nf4.quantize(W)
    assert packed[0] == 0x0F and packed[1] == 0xF0


def test_storage_closed_form():
    for N, K in [(1024, 1024), (4096, 4096), (22016, 8192), (8192, 22016), (5120, 13824)]:
        nb = N * K // 64
        b = nf4.storage_bytes(N, K)
        assert b == N * K // 2 + nb + 4 * math.ceil(nb / 256)
        bits = 8 * b / (N * K)
        assert abs(bits - (4 + 8 / 64 + 32 / 16384)) < 1e-3
    # about 4x smaller than 16 bits, about 75% less memory
    bits = 4 + 8 / 64 + 32 / 16384
    assert 3.8 < 16 / bits < 4.0
    assert 0.73 < 1 - bits / 16 < 0.76


def test_quantizer_output_sizes():
    W = np.random.default_rng(0).standard_normal((3, 1024 * 8)).astype(np.float32)
    packed, q8, step = nf4.quantize(W)
    assert packed.size == 3 * 8192 // 2 and q8.size == 3 * 8192 // 64
    assert step.size == math.ceil(3 * 8192 / 64 / 256)
    assert packed.size + q8.size + 4 * step.size == nf4.storage_bytes(3, 8192)


def _tiny_fixture():
    path = __file__.replace("test_oracle_nf4.py", "golden/nf4_tiny_2x128.txt")
    rows = {}
    for line in open(path):
        if line.startswith("#"):
            continue
        key, rest = line.split(" ", 1)
        rows[key] = rest.split()
    W = np.array([int(t, 16) for t in rows["W"]], np.uint32).view(np.float32).reshape(2, 128)
    codes = np.frombuffer(bytes.fromhex(rows["codes"][0]), np.uint8)
    q8 = np.frombuffer(bytes.fromhex(rows["q8"][0]), np.uint8)
    step = np.array([int(t, 16) for t in rows["step"]], np.uint32)
    deq = np.array([int(t, 16) for t in rows["deq"]], np.uint16).reshape(2, 128)
    return W, codes, q8, step, deq


def test_tiny_fixture_is_reproduced_by_the_scalar_quantizer():
    """The stored 2x128 fixture (written by the vectorized oracle) against the
    element-by-element pure-Python quantizer and dequantizer: two independent
    codings of the same definition agree bit for bit."""
    W, codes, q8, step, deq = _tiny_fixture()
    sc, sq, ss = scalar.quantize(W.tolist(), [float(v) for v in LEVELS])
    assert bytes(sc) == codes.tobytes()
    assert list(sq) == q8.tolist()
    assert [scalar.f32_bits(v) for v in ss] == step.tolist()
    sd = scalar.dequantize(sc, sq, ss, [float(v) for v in LEVELS])
    assert list(sd) == deq.reshape(-1).tolist()
    # and the vectorized oracle as it stands today
    pc, pq, ps = nf4.quantize(W)
    assert np.array_equal(pc, codes) and np.array_equal(pq, q8)
    assert np.array_equal(ps.view(np.uint32), step)
    assert np.array_equal(nf4.dequantize(pc, pq, ps, 2, 128), deq)
