"""GPU parity of the caller-codebook code types (user4, user3, user2)
through the C ABI, against the CPU oracle.

The ModuLoRA abstract finetunes through weights materialized from a
black-box quantizer, so the layer takes any 2^k values behind the codes:
the library derives the quantizer's thresholds on the host and hands the
values to every kernel in its arguments.  Checks: the quantizer and
dequantizer bit-exact for codebooks of every kind (plain, with zero,
repeated values, zero-free symmetric, values one ulp apart) on random and
adversarial weights; a built-in table passed as a codebook reproduces the
built-in type's state and layer output bit for bit (the run-time table path
equals the compile-time one); the layer within gpu_util's tolerances on
both forward paths and at block sizes 64 and 256; the tile path on an
identity input bit-exact.
"""

import numpy as np
import pytest
import torch

import quantized_base_lora_nf4_amd as qn
from oracle import linear, nf4
from workloads import CODEBOOK_KINDS, draw_codebook, draw_layer, rng_for, to_bf16_bits
from gpu_util import assert_close, dev_u16, f32, host_u16, nf4_host, say

pytestmark = pytest.mark.gpu

USER = ["user4", "user3", "user2"]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    qn.lib()


def _quant(W, code, levels, bs=64):
    w = qn.nf4_quantize(torch.from_numpy(np.ascontiguousarray(W, np.float32)).cuda(), code=code,
                        levels=levels, blocksize=bs)
    torch.cuda.synchronize()
    return w


def _check_quant(W, code, levels, tag, bs=64):
    say(f"[{code} quantize] {tag} {W.shape} bs={bs}")
    w = _quant(W, code, levels, bs)
    codes, q8, step = nf4_host(w)
    oc, oq, os_ = nf4.quantize(W, blocksize=bs, code=code, levels=levels)
    assert np.array_equal(codes, oc), f"{tag}: codes differ at {np.nonzero(codes != oc)[0][:8]}"
    assert np.array_equal(q8, oq), f"{tag}: q8 differ"
    assert np.array_equal(step.view(np.uint32), os_.view(np.uint32)), f"{tag}: steps differ"
    deq = host_u16(qn.nf4_dequantize(w))
    od = nf4.dequantize(oc, oq, os_, *W.shape, blocksize=bs, code=code, levels=levels)
    assert np.array_equal(deq, od), f"{tag}: dequantized bits differ"


def _adversarial(levels, rng):
    """Rows whose normalized values sit on and beside every midpoint of the
    codebook (each row's first element is 1 so the block constant is 1),
    plus a zero row, signed zeros and tiny values."""
    d = sorted(set(float(v) for v in levels))
    pts = []
    for a, b in zip(d[:-1], d[1:]):
        f = np.float32((a + b) / 2)
        pts += [f, np.nextafter(f, np.float32(-2)), np.nextafter(f, np.float32(2))]
    pts = [p for p in pts if -1.0 <= float(p) <= 1.0]
    pts += [0.0, -0.0, 1e-45, -1e-45, 1e-30, -1e-30]
    row = np.zeros(64 * ((len(pts) + 1 + 63) // 64), np.float32)
    row[0] = 1.0
    row[1:1 + len(pts)] = pts
    rows = [row, -row, np.zeros_like(row)]
    noise = (rng.standard_normal(row.size) * 0.3).clip(-1, 1).astype(np.float32)
    noise[0] = 1.0
    rows.append(noise)
    return np.stack(rows).astype(np.float32)


@pytest.mark.parametrize("code", USER)
@pytest.mark.parametrize("kind", CODEBOOK_KINDS)
def test_quantize_dequantize_bitexact(code, kind):
    rng = rng_for(500 + USER.index(code), CODEBOOK_KINDS.index(kind))
    levels = draw_codebook(rng, nf4.CODE_BITS[code], kind)
    W = (rng.standard_normal((33, 1024 + 64)) * 0.02).astype(np.float32)
    W[rng.random(W.shape) < 0.01] *= 10
    _check_quant(W, code, levels, f"{kind} random")
    _check_quant(_adversarial(levels, rng), code, levels, f"{kind} midpoints")


@pytest.mark.parametrize("code", USER)
def test_block_size_256_bitexact(code):
    rng = rng_for(510, USER.index(code))
    levels = draw_codebook(rng, nf4.CODE_BITS[code], "with_zero")
    W = (rng.standard_normal((9, 2048)) * 0.02).astype(np.float32)
    _check_quant(W, code, levels, "random", bs=256)


@pytest.mark.parametrize("builtin,user", [("nf4", "user4"), ("fp4", "user4"),
                                          ("nf3", "user3"), ("nf2", "user2")])
@pytest.mark.parametrize("M", [4, 256])
def test_builtin_table_as_codebook_is_bit_identical(builtin, user, M):
    """The same values through the run-time table give the same state and,
    on both forward paths, the same Y and dX bit for bit."""
    N, K, r = 520, 1088, 16
    inp = draw_layer(N, K, M, r, 2.0, seed=11, index=M)
    lv, _ = qn.code_table(builtin)
    wb = qn.nf4_quantize(torch.from_numpy(inp.W).cuda(), code=builtin)
    wu = qn.nf4_quantize(torch.from_numpy(inp.W).cuda(), code=user, levels=lv)
    for a, b in zip(nf4_host(wb), nf4_host(wu)):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
    X, A, B, dY = dev_u16(inp.X), dev_u16(inp.A), dev_u16(inp.B), dev_u16(inp.dY)
    Yb = qn.qlora_linear_fwd(wb, X, A, B, inp.s)
    Yu = qn.qlora_linear_fwd(wu, X, A, B, inp.s)
    dXb = qn.qlora_linear_bwd(wb, X, dY, A, B, inp.s)[0]
    dXu = qn.qlora_linear_bwd(wu, X, dY, A, B, inp.s)[0]
    torch.cuda.synchronize()
    assert torch.equal(Yb, Yu) and torch.equal(dXb, dXu)


@pytest.mark.parametrize("code", ["user4", "user2"])
@pytest.mark.parametrize("bs", [64, 256])
def test_identity_input_returns_dequantized_weight_bitexact(code, bs):
    N, K, r, M = 136, 5 * bs, 8, 136
    rng = rng_for(520, bs)
    levels = draw_codebook(rng, nf4.CODE_BITS[code], "plain")
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    w = _quant(W, code, levels, bs)
    X = dev_u16(to_bf16_bits(np.eye(K, dtype=np.float32)[:M]))
    A = dev_u16(to_bf16_bits(np.ones((r, K), np.float32) * 0.01))
    B = torch.zeros(N, r, dtype=torch.int16, device="cuda")
    Y = qn.qlora_linear_fwd(w, X, A, B, 2.0)
    ref = nf4.dequantize(*nf4.quantize(W, blocksize=bs, code=code, levels=levels), N, K,
                         blocksize=bs, code=code, levels=levels)
    assert np.array_equal(host_u16(Y), np.ascontiguousarray(ref.T[:M]))


@pytest.mark.parametrize("code", USER)
@pytest.mark.parametrize("shape", [(256, 1024, 1024, 8), (513, 520, 1280, 72), (1, 1024, 2048, 16),
                                   (16, 1032, 1280, 16), (4, 28672, 256, 8)])
@pytest.mark.parametrize("bs", [64, 256])
def test_layer_parity(code, shape, bs):
    M, N, K, r = shape
    say(f"[{code} layer] M={M} N={N} K={K} r={r} bs={bs}")
    rng = rng_for(530 + bs, M + N + K + r)
    levels = draw_codebook(rng, nf4.CODE_BITS[code], "plain")
    inp = draw_layer(N, K, M, r, 2.0, seed=12, index=M + N + K + r + bs)
    w = _quant(inp.W, code, levels, bs)
    X, A, B, dY = dev_u16(inp.X), dev_u16(inp.A), dev_u16(inp.B), dev_u16(inp.dY)
    U = torch.empty(M, r, dtype=torch.int16, device="cuda")
    Y = qn.qlora_linear_fwd(w, X, A, B, inp.s, U_out=U)
    dX, dA, dB = qn.qlora_linear_bwd(w, X, dY, A, B, inp.s, U=U)
    torch.cuda.synchronize()
    Wh = f32(nf4.dequantize(*nf4.quantize(inp.W, blocksize=bs, code=code, levels=levels), N, K,
                            blocksize=bs, code=code, levels=levels))
    Xf, Af, Bf, dYf = f32(inp.X), f32(inp.A), f32(inp.B), f32(inp.dY)
    assert_close("Y", f32(host_u16(Y)), linear.forward(Xf, Wh, Af, Bf, inp.s))
    rdX, rdA, rdB = linear.backward(Xf, dYf, Wh, Af, Bf, inp.s)
    assert_close("dX", f32(host_u16(dX)), rdX)
    assert_close("dA", f32(host_u16(dA)), rdA)
    assert_close("dB", f32(host_u16(dB)), rdB)
