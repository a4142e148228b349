"""The forward entry point that allocates nothing (qlora_linear_fwd_noalloc,
for callers that cannot call hipMalloc) against the plain forward, called
through the C ABI: two calls in a row on the library's fixed scratch, the
second with a smaller input, each bit-identical to qlora_linear_fwd on the
same inputs (same kernels, same workspace layout) and within the layer
tolerance of the oracle (max|d|/max|ref| <= 2e-2, fp64 reference)."""

import numpy as np
import pytest
import torch

import quantized_base_lora_nf4_amd as qn
from oracle import linear
from gpu_util import assert_close, dev_u16, f32, gpu_quantize, host_u16, oracle_what, say
from workloads import draw_layer

pytestmark = pytest.mark.gpu

# (M, N, K, r): first call, then a smaller one
PAIRS = [
    [(2048, 4096, 4096, 64), (300, 520, 1088, 8)],    # tile path, then a smaller tile-path call
    [(16, 4096, 4096, 16), (1, 1024, 2048, 8)],       # few-token path twice
    [(700, 1032, 2048, 128), (4, 136, 192, 4)],       # tile path, then few-token
]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    qn.lib()


def _run(shape, seed):
    M, N, K, r = shape
    inp = draw_layer(N, K, M, r, 2.0, seed=seed, index=M + N + K + r)
    w = gpu_quantize(inp.W)
    X, A, B = dev_u16(inp.X), dev_u16(inp.A), dev_u16(inp.B)
    Y0 = torch.empty(M, N, dtype=torch.int16, device="cuda")
    U0 = torch.empty(M, r, dtype=torch.int16, device="cuda")
    Y1 = torch.full((M, N), -1, dtype=torch.int16, device="cuda")
    U1 = torch.full((M, r), -1, dtype=torch.int16, device="cuda")
    qn.qlora_linear_fwd(w, X, A, B, inp.s, Y=Y0, U_out=U0)
    qn.qlora_linear_fwd_noalloc(w, X, A, B, inp.s, Y=Y1, U_out=U1)
    torch.cuda.synchronize()
    return inp, (host_u16(Y0), host_u16(U0)), (host_u16(Y1), host_u16(U1))


@pytest.mark.parametrize("pair", PAIRS, ids=lambda p: f"{p[0]}-then-{p[1]}")
def test_noalloc_forward_matches_the_plain_forward_twice_in_a_row(pair):
    for i, shape in enumerate(pair):
        say(f"[no-alloc] call {i}: M,N,K,r = {shape}")
        inp, (y0, u0), (y1, u1) = _run(shape, seed=i)
        assert np.array_equal(y0, y1), f"call {i}: Y differs from qlora_linear_fwd"
        assert np.array_equal(u0, u1), f"call {i}: U differs from qlora_linear_fwd"
        What = oracle_what(inp.W)
        X, A, B = f32(inp.X), f32(inp.A), f32(inp.B)
        assert_close("Y", f32(y1), linear.forward(X, What, A, B, inp.s))
        assert_close("U", f32(u1), linear.lora_down(X, A))


def test_noalloc_forward_rejects_a_call_past_its_scratch():
    M, N, K, r = 1 << 16, 64, 128, 256   # U alone is 32 MiB
    assert qn.workspace_size(M, N, K, r, False) > qn._lib.QLORA_NOALLOC_SCRATCH_BYTES
    w = qn.alloc_nf4(N, K)
    X = torch.zeros(M, K, dtype=torch.bfloat16, device="cuda")
    A = torch.zeros(r, K, dtype=torch.bfloat16, device="cuda")
    B = torch.zeros(N, r, dtype=torch.bfloat16, device="cuda")
    Y = torch.zeros(M, N, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(qn.QloraError, match="workspace"):
        qn.qlora_linear_fwd_noalloc(w, X, A, B, 1.0, Y=Y)
