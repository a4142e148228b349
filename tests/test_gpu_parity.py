"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bit-exact: packed codes, 8-bit constants, fp32 steps, dequantized bf16.
Tolerance (max|d| / max|ref| <= 2e-2 per tensor, fp64 reference, written
in gpu_util.TOL): Y, dX, dA, dB.

Shapes span several tiles with ragged tails in every dimension; special
inputs cover all-zero weights, subnormal blocks, ties and heavy tails.
"""

import numpy as np
import pytest
import torch

import quantized_base_lora_nf4_amd as qn
from oracle import linear, nf4
from workloads import draw_layer, rng_for, to_bf16_bits
from gpu_util import (TOL, assert_close, dev_u16, f32, gpu_quantize, host_u16, nf4_host,
                      oracle_what, rel_err, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    qn.lib()  # raises if the HIP library is missing


# ------------------------------------------------------------------ quantizer

def _special_weights():
    rng = np.random.default_rng(11)
    L = nf4.nf4_levels().astype(np.float64)
    out = {}
    out["zeros"] = np.zeros((4, 256), np.float32)
    d = (rng.standard_normal((2, 128)) * 1e-39).astype(np.float32)
    out["subnormal"] = d
    one = np.zeros((3, 64), np.float32)
    one[0, 17] = -0.3
    one[2, 63] = 1e-30
    out["single_nonzero"] = one
    tie = []
    for i in range(15):
        mid = (L[i] + L[i + 1]) / 2
        f = np.float32(mid)
        lo = f if float(f) <= mid else np.nextafter(f, np.float32(-np.inf))
        tie += [lo, np.nextafter(lo, np.float32(np.inf))]
    tie += [1.0, -1.0]
    out["transition_points"] = np.array([tie + tie[::-1]] * 2, np.float32) * np.float32(0.5)
    # the same values in blocks whose absmax sits at and past the ends of the
    # quantizer's refined-division range (2^-60 .. 2^126): IEEE division there
    tp = np.array([tie + tie[::-1]], np.float64)
    out["transition_points_scaled"] = np.concatenate(
        [tp * 2.0 ** e for e in (126, 127, -60, -61, -75, -100)]).astype(np.float32)
    row = np.tile(nf4.nf4_levels() * np.float32(2.0 ** -5), 4)
    out["levels_in_order"] = row[None, :].astype(np.float32)
    w = np.zeros((1, 64 * 4), np.float32)
    w[0, 0] = 255 * 2.0 ** -7
    w[0, 64:128] = 0.001
    out["pow2_group_max"] = w
    h = (rng.standard_normal((8, 2048)) * 0.02).astype(np.float32)
    h[rng.random(h.shape) < 0.01] *= 10
    out["heavy_tail"] = h
    return out


QSHAPES = [(1, 64), (2, 128), (3, 1024), (5, 4096), (7, 192), (64, 4096), (1000, 1024),
           (33, 8192 + 64)]


def _check_quant(W, tag):
    say(f"[quantize] {tag} {W.shape}")
    w = gpu_quantize(W)
    codes, q8, step = nf4_host(w)
    oc, oq, os_ = nf4.quantize(W)
    assert np.array_equal(codes, oc), f"{tag}: codes differ at {np.nonzero(codes != oc)[0][:8]}"
    assert np.array_equal(q8, oq), f"{tag}: q8 differ at {np.nonzero(q8 != oq)[0][:8]}"
    assert np.array_equal(step.view(np.uint32), os_.view(np.uint32)), f"{tag}: steps differ"
    deq = host_u16(qn.nf4_dequantize(w))
    od = nf4.dequantize(oc, oq, os_, *W.shape)
    assert np.array_equal(deq, od), f"{tag}: dequantized bits differ at {np.argwhere(deq != od)[:8]}"


@pytest.mark.parametrize("shape", QSHAPES)
def test_quantize_dequantize_bitexact_random(shape):
    rng = rng_for(100, shape[0] * 100000 + shape[1])
    W = (rng.standard_normal(shape) * 0.02).astype(np.float32)
    _check_quant(W, "random")


@pytest.mark.parametrize("name", list(_special_weights().keys()))
def test_quantize_dequantize_bitexact_special(name):
    _check_quant(_special_weights()[name], name)


def test_quantize_is_deterministic():
    W = (np.random.default_rng(5).standard_normal((96, 2048)) * 0.02).astype(np.float32)
    a = nf4_host(gpu_quantize(W))
    b = nf4_host(gpu_quantize(W))
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8))


# ------------------------------------------------------------------ layer

LSHAPES = [  # (M, N, K, r)
    (256, 1024, 1024, 8),      # the 1024 x 1024 workload
    (300, 136, 192, 8),        # ragged M, N and K against the 256 x 128 tiles
    (17, 264, 320, 5),         # smallest tile path, odd rank
    (513, 520, 1088, 72),      # rank above 64: two LoRA steps
    (64, 64, 64, 1),
    (1, 1024, 2048, 16),       # few-token path
    (4, 1024, 2048, 16),
    (16, 1032, 1024, 16),
    (16, 8, 64, 3),
    (9, 2056, 4160, 64),
    (300, 264, 512, 256),      # the largest rank: four LoRA steps, padded U
    (4, 1024, 2048, 256),      # the largest rank on the few-token path
    (130, 520, 576, 128),      # rank 128, ragged M and N
    (2, 8, 64, 1),             # one block per weight row, smallest everything
    (260, 392, 768, 16),       # K % 256 == 0 with 12 steps: grouped constants plus a tail group
    (33, 64, 256, 4),          # K = 256: the tail group alone
    # 28672 rows = 7 x 16 rows per CU on a 256-CU device: the few-token
    # forward takes workgroups of 7 row groups there
    (3, 28672, 64, 4),         # one block per row: the odd tail step alone
    (16, 28672, 192, 16),      # three blocks: one double step and the tail
    (7, 28672, 576, 8),
    (5, 28672, 2560, 16),      # 20 double steps: partial chunks of the row-group-major loop
    (2, 1000, 1088, 8),        # two tokens: one row group per workgroup, ragged rows, odd block count
    (3, 64, 41024, 4),         # few tokens, K past the few-token kernel's LDS tables: tile path
    (70000, 136, 192, 8),      # 274 row tiles (ragged, not a multiple of 8): the XCD tile order's
                               # remainder, and 70000-long contractions for dA and dB
]


def _layer(M, N, K, r, seed=0, s=None):
    s = 2.0 if s is None else s
    return draw_layer(N, K, M, r, s, seed=seed, index=M + N + K + r)


def _gpu_fwd_bwd(inp, w, with_bwd=True, give_u=True):
    X, A, B = dev_u16(inp.X), dev_u16(inp.A), dev_u16(inp.B)
    M, r = inp.X.shape[0], inp.A.shape[0]
    U = torch.empty(M, r, dtype=torch.int16, device="cuda") if give_u else None
    Y = torch.empty(M, w.N, dtype=torch.int16, device="cuda")
    qn.qlora_linear_fwd(w, X, A, B, inp.s, Y=Y, U_out=U)
    res = {"Y": f32(host_u16(Y))}
    if with_bwd:
        dY = dev_u16(inp.dY)
        dX, dA, dB = qn.qlora_linear_bwd(w, X, dY, A, B, inp.s, U=U if give_u else None)
        res.update(dX=f32(host_u16(dX)), dA=f32(host_u16(dA)), dB=f32(host_u16(dB)))
    if give_u:
        res["U"] = f32(host_u16(U))
    torch.cuda.synchronize()
    return res


@pytest.mark.parametrize("shape", LSHAPES)
def test_layer_parity(shape):
    M, N, K, r = shape
    say(f"[layer] M={M} N={N} K={K} r={r}")
    inp = _layer(M, N, K, r)
    w = gpu_quantize(inp.W)
    got = _gpu_fwd_bwd(inp, w)
    Wh = oracle_what(inp.W)
    X, A, B, dY = f32(inp.X), f32(inp.A), f32(inp.B), f32(inp.dY)
    assert_close("Y", got["Y"], linear.forward(X, Wh, A, B, inp.s))
    assert_close("U", got["U"], linear.lora_down(X, A))
    dX, dA, dB = linear.backward(X, dY, Wh, A, B, inp.s)
    assert_close("dX", got["dX"], dX)
    assert_close("dA", got["dA"], dA)
    assert_close("dB", got["dB"], dB)


@pytest.mark.parametrize("shape", [(3, 8, 1 << 22, 2),     # K = QLORA_LINEAR_MAX_NK: 8 MB rows
                                   (2, 1 << 22, 64, 1)])   # N = QLORA_LINEAR_MAX_NK
def test_layer_parity_at_the_largest_N_and_K(shape):
    """The largest N and K the layer calls accept: every 32-bit offset the
    kernels form (a 256-row tile of 8 MB rows spans just under 2 GiB) and
    the tile path a few tokens take when K is past the few-token kernel's
    tables."""
    M, N, K, r = shape
    say(f"[layer max] M={M} N={N} K={K} r={r}")
    inp = _layer(M, N, K, r)
    w = gpu_quantize(inp.W)
    got = _gpu_fwd_bwd(inp, w)
    Wh = oracle_what(inp.W)
    X, A, B, dY = f32(inp.X), f32(inp.A), f32(inp.B), f32(inp.dY)
    assert_close("Y", got["Y"], linear.forward(X, Wh, A, B, inp.s))
    assert_close("U", got["U"], linear.lora_down(X, A))
    dX, dA, dB = linear.backward(X, dY, Wh, A, B, inp.s)
    assert_close("dX", got["dX"], dX)
    assert_close("dA", got["dA"], dA)
    assert_close("dB", got["dB"], dB)


def _poisoned_copy(w, rows=64):
    """The same weight state at the start of larger buffers whose bytes past
    the end hold garbage (codes 0xFF, constants 255, steps NaN), `rows`
    weight rows' worth of each.  A kernel that reads any of it for a row past
    N puts NaN or huge values into its results."""
    kb = w.K // 64
    def pad(t, extra, fill):
        big = torch.full((t.numel() + extra,), fill, dtype=t.dtype, device=t.device)
        big[:t.numel()].copy_(t)
        return big[:t.numel()]
    return qn.NF4Weight(codes=pad(w.codes, rows * w.codes.numel() // w.N, 0xFF),
                        q8=pad(w.q8, rows * kb, 0xFF),
                        step=pad(w.step, rows * kb // 256 + 2, float("nan")),
                        N=w.N, K=w.K, code=w.code)


@pytest.mark.parametrize("shape", [(300, 136, 192, 8), (260, 392, 768, 16), (130, 520, 576, 128),
                                   (16, 1032, 1024, 16)])
def test_layer_reads_nothing_past_the_weight(shape):
    """N not a multiple of 64: the backward's last contraction step covers
    weight rows past N, which must contribute exactly zero without reading
    memory past the weight's buffers (garbage is planted there)."""
    M, N, K, r = shape
    say(f"[poisoned tail] M={M} N={N} K={K} r={r}")
    inp = _layer(M, N, K, r, seed=5)
    w = _poisoned_copy(gpu_quantize(inp.W))
    got = _gpu_fwd_bwd(inp, w)
    Wh = oracle_what(inp.W)
    X, A, B, dY = f32(inp.X), f32(inp.A), f32(inp.B), f32(inp.dY)
    assert_close("Y", got["Y"], linear.forward(X, Wh, A, B, inp.s))
    dX, dA, dB = linear.backward(X, dY, Wh, A, B, inp.s)
    assert_close("dX", got["dX"], dX)
    assert_close("dA", got["dA"], dA)
    assert_close("dB", got["dB"], dB)


@pytest.mark.parametrize("shape", [(300, 136, 192, 8), (4, 1024, 2048, 16), (257, 512, 512, 64)])
def test_lora_terms_in_isolation(shape):
    """W = 0 leaves only the adapter: Y = s U B^T, dX = s dY B A.  The LoRA
    term is ~1-3 % of Y in the real workloads, so it is checked alone."""
    M, N, K, r = shape
    say(f"[lora-only] {shape}")
    inp = _layer(M, N, K, r, s=0.75)
    inp.W[:] = 0
    w = gpu_quantize(inp.W)
    got = _gpu_fwd_bwd(inp, w)
    X, A, B, dY = f32(inp.X), f32(inp.A), f32(inp.B), f32(inp.dY)
    Z = np.zeros((N, K))
    assert_close("Y", got["Y"], linear.forward(X, Z, A, B, inp.s))
    dX, dA, dB = linear.backward(X, dY, Z, A, B, inp.s)
    assert_close("dX", got["dX"], dX)
    assert_close("dA", got["dA"], dA)
    assert_close("dB", got["dB"], dB)


def test_identity_input_returns_dequantized_weight_bitexact():
    """X = I_K with B = 0: the tile path writes W_hat^T exactly (every
    product is 1 * w or 0 * w, every sum has one non-zero term)."""
    N, K, r = 136, 320, 8
    say("[identity]")
    W = (np.random.default_rng(3).standard_normal((N, K)) * 0.02).astype(np.float32)
    w = gpu_quantize(W)
    X = dev_u16(to_bf16_bits(np.eye(K, dtype=np.float32)))
    A = dev_u16(to_bf16_bits(np.ones((r, K), np.float32) * 0.01))
    B = torch.zeros(N, r, dtype=torch.int16, device="cuda")
    Y = qn.qlora_linear_fwd(w, X, A, B, 2.0)
    ref = nf4.dequantize(*nf4.quantize(W), N, K)
    assert np.array_equal(host_u16(Y), np.ascontiguousarray(ref.T))


def test_backward_without_dx_and_without_saved_u():
    M, N, K, r = 100, 256, 512, 16
    inp = _layer(M, N, K, r)
    w = gpu_quantize(inp.W)
    X, A, B, dY = dev_u16(inp.X), dev_u16(inp.A), dev_u16(inp.B), dev_u16(inp.dY)
    dX, dA, dB = qn.qlora_linear_bwd(w, X, dY, A, B, inp.s, U=None, need_dX=False)
    assert dX is None
    Wh = oracle_what(inp.W)
    _, rdA, rdB = linear.backward(f32(inp.X), f32(inp.dY), Wh, f32(inp.A), f32(inp.B), inp.s)
    assert_close("dA", f32(host_u16(dA)), rdA)
    assert_close("dB", f32(host_u16(dB)), rdB)


@pytest.mark.parametrize("shape", [(300, 520, 1088, 16),   # tile path
                                   (4, 28672, 192, 8),     # few tokens, 7 row groups per workgroup
                                   (1, 1024, 2048, 16)])   # few tokens, 1 row group per workgroup
def test_layer_is_deterministic(shape):
    inp = _layer(*shape)
    w = gpu_quantize(inp.W)
    a = _gpu_fwd_bwd(inp, w)
    b = _gpu_fwd_bwd(inp, w)
    for k in a:
        assert np.array_equal(a[k].view(np.uint32), b[k].view(np.uint32)), k


@pytest.mark.parametrize("shape", [(300, 520, 1088, 16), (4, 1024, 2048, 16)])
def test_layer_on_a_side_stream_matches_the_default_stream(shape):
    """Every launch goes to the stream the caller passes (here torch's
    current stream inside a stream context): bit-identical results."""
    inp = _layer(*shape)
    w = gpu_quantize(inp.W)
    a = _gpu_fwd_bwd(inp, w)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        b = _gpu_fwd_bwd(inp, w)
    torch.cuda.synchronize()
    for k in a:
        assert np.array_equal(a[k].view(np.uint32), b[k].view(np.uint32)), k


def test_autograd_function_matches_direct_calls():
    M, N, K, r = 64, 128, 256, 8
    inp = _layer(M, N, K, r)
    Wd = torch.from_numpy(inp.W).cuda()
    lay = qn.QLoRALinear(Wd, r, alpha=16.0,
                         A=dev_u16(inp.A).view(torch.bfloat16), B=dev_u16(inp.B).view(torch.bfloat16))
    X = dev_u16(inp.X).view(torch.bfloat16).requires_grad_(True)
    Y = lay(X)
    Y.backward(dev_u16(inp.dY).view(torch.bfloat16))
    Wh = oracle_what(inp.W)
    s = 16.0 / r
    ref_Y = linear.forward(f32(inp.X), Wh, f32(inp.A), f32(inp.B), s)
    dX, dA, dB = linear.backward(f32(inp.X), f32(inp.dY), Wh, f32(inp.A), f32(inp.B), s)
    assert_close("Y", Y.detach().float().cpu().numpy(), ref_Y)
    assert_close("dX", X.grad.float().cpu().numpy(), dX)
    assert_close("dA", lay.A.grad.float().cpu().numpy(), dA)
    assert_close("dB", lay.B.grad.float().cpu().numpy(), dB)


def test_quantizer_reproduces_the_stored_tiny_fixture():
    """tests/golden/nf4_tiny_2x128.txt (written by the oracle's script):
    codes, constants, step and dequantized bits of a hand-built 2x128 weight
    with a zero, a sine ramp, periodic 5x spikes and one -0.25 outlier."""
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "nf4_tiny_2x128.txt")
    rows = {l.split(" ", 1)[0]: l.split()[1:] for l in open(path) if not l.startswith("#")}
    W = np.array([int(t, 16) for t in rows["W"]], np.uint32).view(np.float32).reshape(2, 128)
    w = gpu_quantize(W)
    codes, q8, step = nf4_host(w)
    assert codes.tobytes().hex() == rows["codes"][0]
    assert q8.tobytes().hex() == rows["q8"][0]
    assert ["%08x" % v for v in step.view(np.uint32)] == rows["step"]
    deq = host_u16(qn.nf4_dequantize(w))
    assert ["%04x" % v for v in deq.reshape(-1)] == rows["deq"]


def test_explicit_stream_argument_allocates_on_that_stream():
    """stream= a side stream (not the current one): the binding allocates Y,
    the gradients and the workspace on that stream, so memory that the
    current stream allocates and fills right after the calls, before any
    synchronization, cannot alias buffers the side stream's kernels still
    use.  Results are bit-identical to the default-stream run."""
    inp = _layer(300, 520, 1088, 16)
    w = gpu_quantize(inp.W)
    ref = _gpu_fwd_bwd(inp, w)
    X, A, B, dY = dev_u16(inp.X), dev_u16(inp.A), dev_u16(inp.B), dev_u16(inp.dY)
    M, r = inp.X.shape[0], inp.A.shape[0]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    U = torch.empty(M, r, dtype=torch.int16, device="cuda")
    U.record_stream(side)
    Y = qn.qlora_linear_fwd(w, X, A, B, inp.s, U_out=U, stream=side)
    dX, dA, dB = qn.qlora_linear_bwd(w, X, dY, A, B, inp.s, U=U, stream=side)
    # the current stream takes and overwrites memory of the same sizes now
    junk = [torch.full((n,), -1, dtype=torch.uint8, device="cuda")
            for n in (qn.workspace_size(M, w.N, w.K, r, True), Y.numel() * 2, dX.numel() * 2,
                      dA.numel() * 2, dB.numel() * 2)]
    torch.cuda.synchronize()
    del junk
    got = {"Y": f32(host_u16(Y)), "U": f32(host_u16(U)), "dX": f32(host_u16(dX)),
           "dA": f32(host_u16(dA)), "dB": f32(host_u16(dB))}
    for k in ref:
        assert np.array_equal(ref[k].view(np.uint32), got[k].view(np.uint32)), k
