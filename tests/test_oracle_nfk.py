"""Pins for the k-bit NormalFloat side of the quantizer oracle (NF3, NF2;
CPU only).

The levels are pinned to an independent construction with scipy's normal
quantile, to the NF4 table at k = 4, and to the equal-share property; the
dense k-bit packing to a pure-Python packer, to its inverse, to its size and
locality, and to the shift-and-mask unpacking of eight codes that the
kernels use; the quantizer to the scalar brute force and to its error bound.
"""

import struct

import numpy as np
import pytest
import scipy.special as sp

from oracle import nf4, scalar
from workloads import draw_weight, WeightSpec, rng_for


def _scipy_levels(k):
    n = 2 ** k
    d = 1 - 0.5 * (1 / (2 * (n - 1)) + 1 / (2 * n))
    z = sp.ndtri(d)
    pos = sp.ndtri(np.linspace(d, 0.5, n // 2 + 1)[:-1]) / z
    neg = -sp.ndtri(np.linspace(d, 0.5, n // 2)[:-1]) / z
    return np.sort(np.concatenate([neg, [0.0], pos]))


@pytest.mark.parametrize("k", [2, 3, 4])
def test_levels_match_independent_scipy_construction(k):
    ours = nf4.nfk_levels_f64(k)
    ref = _scipy_levels(k)
    np.testing.assert_allclose(ours, ref, rtol=0, atol=1e-14)
    assert np.array_equal(nf4.nfk_levels(k).view(np.uint32), ref.astype(np.float32).view(np.uint32))


def test_four_bit_case_is_nf4():
    assert np.array_equal(nf4.nfk_levels(4).view(np.uint32), nf4.nf4_levels().view(np.uint32))
    assert nf4.nfk_delta(4) == nf4.NF4_DELTA


@pytest.mark.parametrize("k", [2, 3])
def test_levels_invariants_and_fp32_margin(k):
    v = nf4.nfk_levels_f64(k)
    n = 2 ** k
    assert v.shape == (n,) and np.all(np.diff(v) > 0)
    assert v[0] == -1.0 and v[-1] == 1.0 and v[n // 2 - 1] == 0.0
    assert np.sum(v < 0) == n // 2 - 1 and np.sum(v > 0) == n // 2
    for x in v:
        if x in (-1.0, 0.0, 1.0):
            continue
        f = np.float32(x)
        up, dn = np.nextafter(f, np.float32(np.inf)), np.nextafter(f, np.float32(-np.inf))
        margin = min(x - (float(f) + float(dn)) / 2, (float(f) + float(up)) / 2 - x) / abs(x)
        assert margin > 1e-9


@pytest.mark.parametrize("k", [2, 3])
def test_levels_cover_equal_shares(k):
    d = nf4.nfk_delta(k)
    half = 2 ** (k - 1)
    p = sp.ndtr(nf4.nfk_levels_f64(k) * sp.ndtri(d))
    pos = p[half:]
    neg = 1.0 - p[:half - 1]
    np.testing.assert_allclose(pos[-1], d, atol=1e-14)
    np.testing.assert_allclose(np.diff(pos), (d - 0.5) / half, atol=1e-13)
    if half - 1 > 1:
        np.testing.assert_allclose(np.diff(neg[::-1]), (d - 0.5) / (half - 1), atol=1e-13)
    np.testing.assert_allclose(neg[0], d, atol=1e-14)


def test_nf2_closed_form():
    # NF2: -1, 0, one inner positive level, +1; delta = 1 - (1/6 + 1/8)/2
    d = 1 - (1 / 6 + 1 / 8) / 2
    inner = sp.ndtri(d - (d - 0.5) / 2) / sp.ndtri(d)
    np.testing.assert_allclose(nf4.nfk_levels_f64(2), [-1.0, 0.0, inner, 1.0], atol=1e-15)


# ---------------------------------------------------------------- packing

@pytest.mark.parametrize("bits", [2, 3])
def test_pack_matches_scalar_and_inverts(bits):
    rng = np.random.default_rng(bits)
    codes = rng.integers(0, 2 ** bits, 64 * 9).astype(np.uint8)
    packed = nf4.pack_codes_k(codes, bits)
    assert packed.size == codes.size * bits // 8
    assert bytes(packed.tobytes()) == scalar.pack_kbit([int(c) for c in codes], bits)
    assert np.array_equal(nf4.unpack_codes_k(packed, bits), codes)
    assert scalar.unpack_kbit(bytes(packed.tobytes()), bits, codes.size) == [int(c) for c in codes]


@pytest.mark.parametrize("bits", [2, 3])
def test_each_code_stays_in_its_half_block(bits):
    for e in (0, 1, 7, 8, 31, 32, 33, 62, 63):
        codes = np.zeros(64, np.uint8)
        codes[e] = 2 ** bits - 1
        packed = nf4.pack_codes_k(codes, bits)
        nz = np.nonzero(packed)[0]
        h = e // 32
        assert np.all((nz >= 4 * bits * h) & (nz < 4 * bits * (h + 1))), (e, nz)
        assert sum(bin(int(b)).count("1") for b in packed) == bits


def _rotr(x, n):
    n %= 32
    return ((x >> n) | (x << (32 - n))) & 0xFFFFFFFF if n else x


@pytest.mark.parametrize("bits", [2, 3])
def test_eight_codes_unpack_by_shifts_and_masks(bits):
    # For 8 consecutive codes 8g..8g+7 of a half: byte i of
    # (even word >> 2g) & 0x03030303, plus bit 2 from (C rotated right by
    # 2g + p) & 0x04040404 for 3 bits, is the code of element 8g + 2i + p.
    rng = np.random.default_rng(10 + bits)
    codes = rng.integers(0, 2 ** bits, 64).astype(np.uint8)
    w = [int(x) for x in nf4.pack_codes_k(codes, bits).view("<u4")]
    for h in range(2):
        for g in range(4):
            for p in range(2):
                sel = (w[bits * h + p] >> (2 * g)) & 0x03030303
                if bits == 3:
                    sel |= _rotr(w[3 * h + 2], 2 * g + p) & 0x04040404
                got = [(sel >> (8 * i)) & 0xFF for i in range(4)]
                want = [int(codes[32 * h + 8 * g + 2 * i + p]) for i in range(4)]
                assert got == want, (h, g, p)


# ---------------------------------------------------------------- quantizer

def _tiny(code):
    rng = np.random.default_rng(30)
    lv = nf4.code_values(code).astype(np.float64)
    cases = {
        "normal": (rng.standard_normal((2, 256)) * 0.02).astype(np.float32),
        "zeros_and_one": np.concatenate([np.zeros((1, 64)), rng.standard_normal((1, 64))],
                                        axis=1).astype(np.float32),
    }
    row = []
    for a, b in zip(lv[:-1], lv[1:]):
        f = np.float32((a + b) / 2)
        lo = f if float(f) <= (a + b) / 2 else np.nextafter(f, np.float32(-np.inf))
        row += [lo, np.nextafter(lo, np.float32(np.inf))]
    row += [1.0, -1.0, -0.0]
    row += [0.0] * (64 - len(row))
    cases["transition_points"] = np.array([row, row[::-1]], np.float32)
    cases["levels"] = np.tile(nf4.code_values(code) * np.float32(2.0 ** -3), 64 // lv.size * 2)[None, :]
    return cases


@pytest.mark.parametrize("code", ["nf3", "nf2"])
@pytest.mark.parametrize("name", ["normal", "zeros_and_one", "transition_points", "levels"])
def test_quantizer_matches_scalar_bruteforce(code, name):
    W = _tiny(code)[name]
    packed, q8, step = nf4.quantize(W, code=code)
    lv = [float(v) for v in nf4.code_values(code)]
    sp_, sq, ss = scalar.quantize(W.tolist(), lv)
    assert bytes(packed.tobytes()) == sp_
    assert list(q8) == sq
    assert [struct.pack("<f", v) for v in step] == [struct.pack("<f", v) for v in ss]
    deq = nf4.dequantize(packed, q8, step, *W.shape, code=code)
    assert list(deq.reshape(-1)) == scalar.dequantize(sp_, sq, ss, lv)


@pytest.mark.parametrize("code,k", [("nf3", 3), ("nf2", 2)])
def test_levels_in_order_give_their_codes(code, k):
    W = _tiny(code)["levels"]
    codes = nf4.unpack_codes_k(nf4.quantize(W, code=code)[0], k)
    assert list(codes) == list(range(2 ** k)) * (W.size // 2 ** k)


@pytest.mark.parametrize("code,k", [("nf3", 3), ("nf2", 2)])
def test_all_zero_weight_uses_the_zero_level(code, k):
    W = np.zeros((2, 128), np.float32)
    packed, q8, step = nf4.quantize(W, code=code)
    assert np.all(nf4.unpack_codes_k(packed, k) == 2 ** (k - 1) - 1)
    assert np.all(q8 == 0) and np.all(step == 0)
    assert np.all(nf4.dequantize(packed, q8, step, 2, 128, code=code) == 0)


@pytest.mark.parametrize("code,k", [("nf3", 3), ("nf2", 2)])
def test_round_trip_error_bound_and_end_codes(code, k):
    W = draw_weight(WeightSpec("w", 64, 1024, 0.02, heavy_frac=0.01), rng_for(8, k))
    packed, q8, step = nf4.quantize(W, code=code)
    codes = nf4.unpack_codes_k(packed, k).reshape(-1, 64)
    Wb = W.reshape(-1, 64)
    j = np.argmax(np.abs(Wb), axis=1)
    sel = codes[np.arange(len(j)), j]
    assert np.all(np.where(Wb[np.arange(len(j)), j] > 0, sel == 2 ** k - 1, sel == 0))
    what = nf4.bf16_bits_to_f32(nf4.dequantize(packed, q8, step, *W.shape, code=code))
    lv = nf4.nfk_levels_f64(k)
    half_gap = np.max(np.diff(lv)) / 2
    c = nf4.block_absmax(W).astype(np.float64)
    st = step.astype(np.float64)[np.arange(c.size) // 256]
    err = np.abs(Wb.astype(np.float64) - what.astype(np.float64).reshape(-1, 64))
    slack = 2.0 ** -9 * np.abs(what.reshape(-1, 64)) + 1e-6 * c[:, None]
    assert np.all(err <= (half_gap * c + 0.5 * st)[:, None] + slack)


def test_storage_bytes_by_width():
    for code, bits in (("nf4", 4), ("fp4", 4), ("nf3", 3), ("nf2", 2)):
        N, K = 96, 4096
        nb = N * K // 64
        assert nf4.storage_bytes(N, K, code=code) == N * K * bits // 8 + nb + 4 * ((nb + 255) // 256)
