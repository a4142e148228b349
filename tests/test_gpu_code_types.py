"""GPU parity of the code types other than NF4 through the C ABI, against
the CPU oracle: FP4 (the E2M1 reading of the pages' "fp4" data type) and the
3- and 2-bit NormalFloat types NF3 and NF2 with their dense packing.

The kernels are the NF4 ones with another code table and, for NF3 and NF2,
another code width, so the checks cover what those change: every code of the
quantizer and its packing (bit-exact, including +0 / -0, exact ties and the
transitions between values), the dequantizer, and the forward and backward
layer on both forward paths (few-token weight streaming and the MFMA tiles).
Tolerance as for NF4 (gpu_util.TOL).
"""

import numpy as np
import pytest
import torch

import quantized_base_lora_nf4_amd as qn
from oracle import linear, nf4
from workloads import draw_layer, rng_for, to_bf16_bits
from gpu_util import assert_close, dev_u16, f32, gpu_quantize, host_u16, nf4_host, oracle_what, say

pytestmark = pytest.mark.gpu

CODES = ["fp4", "nf3", "nf2"]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    qn.lib()


def _check_quant(W, tag, code):
    say(f"[{code} quantize] {tag} {W.shape}")
    w = gpu_quantize(W, code=code)
    assert w.code == code
    codes, q8, step = nf4_host(w)
    oc, oq, os_ = nf4.quantize(W, code=code)
    assert np.array_equal(codes, oc), f"{tag}: codes differ at {np.nonzero(codes != oc)[0][:8]}"
    assert np.array_equal(q8, oq), f"{tag}: q8 differ"
    assert np.array_equal(step.view(np.uint32), os_.view(np.uint32)), f"{tag}: steps differ"
    deq = host_u16(qn.nf4_dequantize(w))
    od = nf4.dequantize(oc, oq, os_, *W.shape, code=code)
    assert np.array_equal(deq, od), f"{tag}: dequantized bits differ at {np.argwhere(deq != od)[:8]}"


def _special(code):
    rng = np.random.default_rng(21)
    V = nf4.code_values(code)
    out = {"zeros": np.zeros((4, 256), np.float32)}
    out["signed_zeros"] = np.array([[0.0, -0.0] * 32 + list(rng.standard_normal(64) * 0.02)],
                                   np.float32)
    vals = sorted(set(float(v) for v in V))
    row = []
    for a, b in zip(vals[:-1], vals[1:]):
        mid = (a + b) / 2
        f = np.float32(mid)
        lo = f if float(f) <= mid else np.nextafter(f, np.float32(-np.inf))
        row += [lo, np.nextafter(lo, np.float32(np.inf))]
    h = np.float32(np.float32(vals[vals.index(0.0) + 1]) / np.float32(2))  # exact ties at zero
    row += [h, -h, 1.0, -1.0]
    row += [0.0] * (64 - len(row))
    out["transition_points"] = np.array([row, row[::-1]], np.float32) * np.float32(0.25)
    out["values_in_order"] = np.tile(V * np.float32(2.0 ** -5), 128 // V.size)[None, :].astype(np.float32)
    out["subnormal"] = (rng.standard_normal((2, 128)) * 1e-39).astype(np.float32)
    hv = (rng.standard_normal((8, 2048)) * 0.02).astype(np.float32)
    hv[rng.random(hv.shape) < 0.01] *= 10
    out["heavy_tail"] = hv
    return out


@pytest.mark.parametrize("code", CODES)
@pytest.mark.parametrize("shape", [(1, 64), (3, 1024), (7, 192), (64, 4096), (33, 8192 + 64)])
def test_quantize_dequantize_bitexact_random(code, shape):
    rng = rng_for(200, shape[0] * 100000 + shape[1])
    _check_quant((rng.standard_normal(shape) * 0.02).astype(np.float32), "random", code)


@pytest.mark.parametrize("code", CODES)
@pytest.mark.parametrize("name", list(_special("nf4").keys()))
def test_quantize_dequantize_bitexact_special(code, name):
    _check_quant(_special(code)[name], name, code)


@pytest.mark.parametrize("code", CODES)
@pytest.mark.parametrize("M", [4, 136])
def test_identity_input_returns_dequantized_weight(code, M):
    """X = rows of I_K with B = 0: Y is rows of W_hat^T.  The tile path
    (M = 136) dequantizes exactly as the dequantizer does, so it matches bit
    for bit.  The few-token path (M = 4) multiplies the bf16 code value by
    the block constant after the product, so its element is the same value
    under a different pair of bf16 roundings: within 2^-7 relative."""
    N, K, r = 136, 320, 8
    say(f"[{code} identity] M={M}")
    W = (np.random.default_rng(4).standard_normal((N, K)) * 0.02).astype(np.float32)
    w = gpu_quantize(W, code=code)
    eye = np.eye(K, dtype=np.float32)[:M]
    X = dev_u16(to_bf16_bits(eye))
    A = dev_u16(to_bf16_bits(np.ones((r, K), np.float32) * 0.01))
    B = torch.zeros(N, r, dtype=torch.int16, device="cuda")
    Y = qn.qlora_linear_fwd(w, X, A, B, 2.0)
    ref = nf4.dequantize(*nf4.quantize(W, code=code), N, K, code=code)
    got = host_u16(Y)
    want = np.ascontiguousarray(ref.T[:M])
    if M > 16:
        assert np.array_equal(got, want)
    else:
        g, r_ = f32(got).astype(np.float64), f32(want).astype(np.float64)
        assert np.all(np.abs(g - r_) <= 2.0 ** -7 * np.abs(r_))


@pytest.mark.parametrize("code", CODES)
@pytest.mark.parametrize("shape", [(256, 1024, 1024, 8), (300, 136, 192, 8), (513, 520, 1088, 72),
                                   (1, 1024, 2048, 16), (16, 1032, 1024, 16), (9, 2056, 4160, 64),
                                   (4, 28672, 192, 8)])
def test_layer_parity(code, shape):
    M, N, K, r = shape
    say(f"[{code} layer] M={M} N={N} K={K} r={r}")
    inp = draw_layer(N, K, M, r, 2.0, seed=7, index=M + N + K + r)
    w = gpu_quantize(inp.W, code=code)
    X, A, B, dY = dev_u16(inp.X), dev_u16(inp.A), dev_u16(inp.B), dev_u16(inp.dY)
    U = torch.empty(M, r, dtype=torch.int16, device="cuda")
    Y = qn.qlora_linear_fwd(w, X, A, B, inp.s, U_out=U)
    dX, dA, dB = qn.qlora_linear_bwd(w, X, dY, A, B, inp.s, U=U)
    torch.cuda.synchronize()
    Wh = oracle_what(inp.W, code=code)
    Xf, Af, Bf, dYf = f32(inp.X), f32(inp.A), f32(inp.B), f32(inp.dY)
    assert_close("Y", f32(host_u16(Y)), linear.forward(Xf, Wh, Af, Bf, inp.s))
    rdX, rdA, rdB = linear.backward(Xf, dYf, Wh, Af, Bf, inp.s)
    assert_close("dX", f32(host_u16(dX)), rdX)
    assert_close("dA", f32(host_u16(dA)), rdA)
    assert_close("dB", f32(host_u16(dB)), rdB)
    # the result differs from the NF4 one: the table really is switched
    assert not np.array_equal(Wh, oracle_what(inp.W, code="nf4"))
