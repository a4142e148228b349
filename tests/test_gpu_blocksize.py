"""GPU parity at block sizes 128 and 256 (one absmax constant per 128 or
256 consecutive weights of a row; the constants are still double quantized
in groups of 256 blocks), for every code type, against the CPU oracle.

The block size is a per-matrix quantization parameter that the LQ-LoRA
paper's memory-budget program chooses along with the bit width (LQ-LoRA,
abstract and the section on mixed-configuration quantization).  What it
changes in the kernels is where a weight's constant is read: the quantizer
reduces the absmax over 2 or 4 sixty-four-element units, and every consumer
(dequantizer, MFMA tiles, few-token weight streaming, the backward tiles,
the error of a configuration) indexes constants by k / blocksize.  Codes
stay packed in 64-element units, so the code layout is the block-64 one.

Bars: quantizer and dequantizer bit-exact; layer outputs within gpu_util's
TOL and FROB_TOL; the tile path on an identity input bit-exact against the
oracle's dequantized weight; configuration errors relative 1e-12.
"""

import numpy as np
import pytest
import torch

import quantized_base_lora_nf4_amd as qn
from oracle import ilp, linear, nf4
from workloads import WeightSpec, draw_layer, draw_weight, rng_for, to_bf16_bits
from gpu_util import assert_close, dev_u16, f32, gpu_quantize, host_u16, nf4_host, oracle_what, say

pytestmark = pytest.mark.gpu

CODES = ["nf4", "fp4", "nf3", "nf2"]
SIZES = [128, 256]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    qn.lib()


def _check_quant(W, tag, code, bs):
    say(f"[{code}/{bs} quantize] {tag} {W.shape}")
    w = gpu_quantize(W, code=code, blocksize=bs)
    assert w.blocksize == bs and w.q8.numel() == W.size // bs
    codes, q8, step = nf4_host(w)
    oc, oq, os_ = nf4.quantize(W, blocksize=bs, code=code)
    assert np.array_equal(codes, oc), f"{tag}: codes differ at {np.nonzero(codes != oc)[0][:8]}"
    assert np.array_equal(q8, oq), f"{tag}: q8 differ at {np.nonzero(q8 != oq)[0][:8]}"
    assert np.array_equal(step.view(np.uint32), os_.view(np.uint32)), f"{tag}: steps differ"
    deq = host_u16(qn.nf4_dequantize(w))
    od = nf4.dequantize(oc, oq, os_, *W.shape, blocksize=bs, code=code)
    assert np.array_equal(deq, od), f"{tag}: dequantized bits differ at {np.argwhere(deq != od)[:8]}"


@pytest.mark.parametrize("bs", SIZES)
@pytest.mark.parametrize("code", CODES)
@pytest.mark.parametrize("shape", [(1, 256), (3, 1280), (7, 768), (64, 4096), (33, 8192 + 256)])
def test_quantize_dequantize_bitexact_random(bs, code, shape):
    rng = rng_for(300 + bs, shape[0] * 100000 + shape[1])
    W = (rng.standard_normal(shape) * 0.02).astype(np.float32)
    W[rng.random(shape) < 0.01] *= 10
    _check_quant(W, "random", code, bs)


@pytest.mark.parametrize("bs", SIZES)
def test_absmax_is_taken_over_the_whole_block(bs):
    """One large weight per block, placed in each 64-element unit in turn: the
    constant is that weight's magnitude for the whole block, so every other
    weight of the block is coded against it (a per-64 reduction would not be)."""
    units = bs // 64
    W = np.full((units, 2 * bs), 0.01, np.float32)
    for i in range(units):
        W[i, 64 * i + 5] = 1.0
        W[i, bs + 64 * i + 17] = -0.5
    _check_quant(W, "spike per block", "nf4", bs)
    _, q8, step = nf4_host(gpu_quantize(W, "nf4", bs))
    assert q8.size == 2 * units


@pytest.mark.parametrize("bs", SIZES)
def test_zero_weight_and_ragged_double_quant_group(bs):
    """N*K/bs not a multiple of 256: the last double-quantization group is short."""
    _check_quant(np.zeros((3, bs * 5), np.float32), "zeros", "nf4", bs)
    rng = rng_for(310, bs)
    _check_quant((rng.standard_normal((5, 300 * bs)) * 0.02).astype(np.float32), "ragged group",
                 "nf3", bs)


@pytest.mark.parametrize("bs", SIZES)
@pytest.mark.parametrize("code", ["nf4", "nf2"])
def test_identity_input_returns_dequantized_weight_bitexact(bs, code):
    """Tile path (M > 16), X = rows of I_K, B = 0: Y is rows of W_hat^T."""
    N, K, r, M = 136, 5 * bs, 8, 136
    say(f"[{code}/{bs} identity] M={M}")
    W = (np.random.default_rng(4).standard_normal((N, K)) * 0.02).astype(np.float32)
    w = gpu_quantize(W, code=code, blocksize=bs)
    X = dev_u16(to_bf16_bits(np.eye(K, dtype=np.float32)[:M]))
    A = dev_u16(to_bf16_bits(np.ones((r, K), np.float32) * 0.01))
    B = torch.zeros(N, r, dtype=torch.int16, device="cuda")
    Y = qn.qlora_linear_fwd(w, X, A, B, 2.0)
    ref = nf4.dequantize(*nf4.quantize(W, blocksize=bs, code=code), N, K, blocksize=bs, code=code)
    assert np.array_equal(host_u16(Y), np.ascontiguousarray(ref.T[:M]))


LAYER_SHAPES = [(256, 1024, 1024, 8), (300, 136, 1280, 8), (513, 520, 2304, 72),
                (1, 1024, 2048, 16), (16, 1032, 1280, 16), (9, 2056, 4352, 64),
                (4, 28672, 256, 8)]


@pytest.mark.parametrize("bs", SIZES)
@pytest.mark.parametrize("code", ["nf4", "nf3"])
@pytest.mark.parametrize("shape", LAYER_SHAPES)
def test_layer_parity(bs, code, shape):
    M, N, K, r = shape
    say(f"[{code}/{bs} layer] M={M} N={N} K={K} r={r}")
    inp = draw_layer(N, K, M, r, 2.0, seed=8, index=M + N + K + r + bs)
    w = gpu_quantize(inp.W, code=code, blocksize=bs)
    X, A, B, dY = dev_u16(inp.X), dev_u16(inp.A), dev_u16(inp.B), dev_u16(inp.dY)
    U = torch.empty(M, r, dtype=torch.int16, device="cuda")
    Y = qn.qlora_linear_fwd(w, X, A, B, inp.s, U_out=U)
    dX, dA, dB = qn.qlora_linear_bwd(w, X, dY, A, B, inp.s, U=U)
    torch.cuda.synchronize()
    Wh = oracle_what(inp.W, code=code, blocksize=bs)
    Xf, Af, Bf, dYf = f32(inp.X), f32(inp.A), f32(inp.B), f32(inp.dY)
    assert_close("Y", f32(host_u16(Y)), linear.forward(Xf, Wh, Af, Bf, inp.s))
    rdX, rdA, rdB = linear.backward(Xf, dYf, Wh, Af, Bf, inp.s)
    assert_close("dX", f32(host_u16(dX)), rdX)
    assert_close("dA", f32(host_u16(dA)), rdA)
    assert_close("dB", f32(host_u16(dB)), rdB)
    # the constants really are shared by the whole block
    assert not np.array_equal(Wh, oracle_what(inp.W, code=code, blocksize=64))


@pytest.mark.parametrize("bs", SIZES)
def test_noalloc_forward_matches_forward(bs):
    M, N, K, r = 4, 1032, 1280, 16
    inp = draw_layer(N, K, M, r, 2.0, seed=9, index=bs)
    w = gpu_quantize(inp.W, blocksize=bs)
    X, A, B = dev_u16(inp.X), dev_u16(inp.A), dev_u16(inp.B)
    Y0 = qn.qlora_linear_fwd(w, X, A, B, inp.s)
    Y1 = torch.empty_like(Y0)
    qn.qlora_linear_fwd_noalloc(w, X, A, B, inp.s, Y1)
    torch.cuda.synchronize()
    assert torch.equal(Y0, Y1)


@pytest.mark.parametrize("code,bs", [c for c in ilp.CONFIGS if c[1] != 64])
@pytest.mark.parametrize("shape", [(1, 256), (7, 768), (300, 1024), (1024, 4352)])
def test_config_error_matches_oracle(code, bs, shape):
    W = draw_weight(WeightSpec("w", *shape, 0.02, heavy_frac=0.01), rng_for(43, shape[0] + bs))
    got = float(qn.quant_error(torch.from_numpy(W).cuda(), code, blocksize=bs).cpu().item())
    want = ilp.quant_error(W, code, blocksize=bs)
    say(f"[ilp] {code}/{bs} {shape}: {got:.10g} vs {want:.10g}")
    assert abs(got - want) <= 1e-12 * want
    assert qn.storage_bytes(*shape, code, bs) == ilp.state_bytes(*shape, code, bs)
