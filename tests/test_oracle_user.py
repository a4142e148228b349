"""Pins for the caller-codebook code types of the quantizer oracle (CPU only).

The ModuLoRA abstract finetunes through weights that a black-box quantizer
produced and the backward pass materializes, so the layer has to accept any
2^k values behind the codes.  The oracle quantizes to such a codebook by the
definition of a nearest value (ties to the lower value, of equal values the
lowest code), written as a count of exact midpoints below x.  Each check
ties it to something other than that formula: exact rational distances,
the built-in code types (already pinned elsewhere) fed through the user
path, the pure-Python scalar quantizer, and invariants (relabelling the
codes, sign symmetry, the all-zero block).
"""

import zlib
from fractions import Fraction

import numpy as np
import pytest

from oracle import nf4, scalar
from workloads import CODEBOOK_KINDS, WeightSpec, draw_codebook, draw_weight, rng_for

BUILTIN_AS_USER = [("nf4", "user4"), ("fp4", "user4"), ("nf3", "user3"), ("nf2", "user2")]


def _codebook(rng, code, kind):
    return draw_codebook(rng, nf4.CODE_BITS[code], kind)


def _exact_nearest(x, values):
    """Code of the nearest value by exact rational distance; ties to the
    lower value, equal values to the lowest code."""
    fx = Fraction(float(x))
    return min(range(len(values)),
               key=lambda c: (abs(fx - Fraction(float(values[c]))), Fraction(float(values[c])), c))


def _probes(values, rng):
    """x values that matter: every exact midpoint and its fp32 neighbours,
    the values themselves, signed zeros, subnormals, random points."""
    d = sorted(set(float(v) for v in values))
    pts = [0.0, -0.0, 1.0, -1.0, 1e-45, -1e-45, 1e-39, -1e-39]
    for a, b in zip(d[:-1], d[1:]):
        m = (a + b) / 2
        f = np.float32(m)
        for g in (f, np.nextafter(f, np.float32(-2)), np.nextafter(f, np.float32(2))):
            if -1.0 <= float(g) <= 1.0:
                pts.append(float(g))
    pts += d
    pts += list(rng.uniform(-1, 1, 200).astype(np.float32))
    return np.array(pts, np.float32)


@pytest.mark.parametrize("code", nf4.USER_CODES)
@pytest.mark.parametrize("kind", CODEBOOK_KINDS)
def test_nearest_code_matches_exact_rational_distances(code, kind):
    rng = np.random.default_rng(zlib.crc32(f"{code}/{kind}".encode()))
    for _ in range(5):
        v = _codebook(rng, code, kind)
        x = _probes(v, rng)
        got = nf4.nearest_code_exact(x, nf4.user_values(code, v))
        want = np.array([_exact_nearest(xi, v) for xi in x], np.uint8)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, f"x={x[bad[:4]]} got {got[bad[:4]]} want {want[bad[:4]]} values {v}"


@pytest.mark.parametrize("builtin,user", BUILTIN_AS_USER)
def test_builtin_tables_through_the_user_path_give_the_same_state(builtin, user):
    W = draw_weight(WeightSpec("w", 24, 1024, 0.02, heavy_frac=0.02), rng_for(90, 1))
    W[3] = 0.0
    W[5, :64] = np.linspace(-1, 1, 64, dtype=np.float32)
    a = nf4.quantize(W, code=builtin)
    b = nf4.quantize(W, code=user, levels=nf4.code_values(builtin))
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("code", nf4.USER_CODES)
def test_scalar_quantizer_agrees_on_ordinary_weights(code):
    """The pure-Python quantizer (fp64 distances, one element at a time)
    through packing, double quantization and dequantization."""
    rng = np.random.default_rng(91)
    v = _codebook(rng, code, "plain")
    W = (rng.standard_normal((3, 128)) * 0.02).astype(np.float32)
    packed, q8, step = nf4.quantize(W, code=code, levels=v)
    sp, sq, ss = scalar.quantize(W.tolist(), [float(t) for t in v])
    assert bytes(packed) == bytes(sp) and list(q8) == sq
    assert np.array_equal(step, np.array(ss, np.float32))
    deq = nf4.dequantize(packed, q8, step, 3, 128, code=code, levels=v)
    assert list(deq.reshape(-1)) == scalar.dequantize(sp, sq, ss, [float(t) for t in v])


@pytest.mark.parametrize("code", nf4.USER_CODES)
def test_relabelling_the_codes_permutes_them_and_keeps_the_weight(code):
    rng = np.random.default_rng(92)
    v = _codebook(rng, code, "with_zero")
    perm = rng.permutation(v.size)           # new code c holds old code perm[c]
    v2 = v[perm]
    W = draw_weight(WeightSpec("w", 8, 512, 0.02, heavy_frac=0.05), rng_for(92, 0))
    p1, q1, s1 = nf4.quantize(W, code=code, levels=v)
    p2, q2, s2 = nf4.quantize(W, code=code, levels=v2)
    bits = nf4.CODE_BITS[code]
    c1 = nf4.unpack_codes_k(p1, bits)
    c2 = nf4.unpack_codes_k(p2, bits)
    inv = np.argsort(perm)
    assert np.array_equal(c2, inv[c1])
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2)
    assert np.array_equal(nf4.dequantize(p1, q1, s1, 8, 512, code=code, levels=v),
                          nf4.dequantize(p2, q2, s2, 8, 512, code=code, levels=v2))


def test_zero_free_symmetric_codebook_decides_by_sign():
    """Values -3/4, -1/4, 1/4, 3/4 (codes 0..3): the midpoint of the middle
    pair is 0, so the sign of x decides however tiny x is, and 0 itself is
    a tie that goes to the lower value."""
    v = np.array([-0.75, -0.25, 0.25, 0.75], np.float32)
    x = np.array([1e-45, -1e-45, 0.0, -0.0, 0.5, -0.5, 0.50000006, -0.49999997], np.float32)
    assert list(nf4.nearest_code_exact(x, v)) == [2, 1, 1, 1, 2, 0, 3, 1]


def test_all_zero_block_takes_the_code_nearest_to_zero():
    W = np.zeros((2, 128), np.float32)
    W[1, 64:] = 0.5                       # second row: one zero block, one nonzero
    v = np.array([0.9, -0.3, 0.2, -1.0], np.float32)   # nearest to 0: 0.2 (code 2)
    packed, q8, step = nf4.quantize(W, code="user2", levels=v)
    codes = nf4.unpack_codes_k(packed, 2).reshape(2, 128)
    assert np.all(codes[0] == 2) and np.all(codes[1, :64] == 2)
    assert np.all(codes[1, 64:] == 0)     # x = 1: nearest 0.9


@pytest.mark.parametrize("bad", [[2.0, 0, 0, 0], [1e-7, 0, 0, 0], [np.nan, 0, 0, 0],
                                 [np.inf, 0, 0, 0], [0.5, 0.25, 0.0]])
def test_codebooks_outside_the_contract_are_refused(bad):
    with pytest.raises(ValueError):
        nf4.user_values("user2", bad)
