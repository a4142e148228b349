"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (forward with the saved U, backward from that U, workspace
from qlora_workspace_size, default stream).

Per weight of every workload:
* packed codes, 8-bit constants, fp32 steps and the dequantized bf16
  weight are compared bit for bit with the oracle over the whole tensor;
* U and (unless forward-only) dA and dB are compared in full;
* Y and dX are compared on a seeded sample of rows (row m of Y and of dX
  depends only on row m of X and of dY), which always includes the first
  and the last row; the few-token workload is compared in full.

Tolerance: max|d| / max|ref| <= 2e-2 per tensor against the fp64 oracle
(gpu_util.TOL).
"""

import numpy as np
import pytest
import torch

import quantized_base_lora_nf4_amd as qn
import workloads as wl_mod
from oracle import linear, nf4
from gpu_util import assert_close, dev_u16, f32, host_u16, nf4_host, say

pytestmark = pytest.mark.gpu

SAMPLE_ROWS = 24


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    qn.lib()


def _cases(fwd_only):
    out = []
    for wl in wl_mod.WORKLOADS:
        if wl.fwd_only != fwd_only:
            continue
        for wi, spec in enumerate(wl.weights):
            out.append(pytest.param(wl, wi, id=f"{wl.name}-{spec.name}-{spec.N}x{spec.K}"))
    return out


def _sample_rows(M, seed):
    if M <= SAMPLE_ROWS + 2:
        return np.arange(M)
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(1, M - 1), size=SAMPLE_ROWS, replace=False)
    return np.unique(np.concatenate([[0, M - 1], mid]))


def _quantize_and_check(W, tag):
    """GPU quantize + dequantize, bit-exact against the oracle over the
    whole weight; returns the GPU weight and the oracle's W_hat (fp32)."""
    N, K = W.shape
    say(f"[fullsize] {tag}: quantize {N}x{K}")
    Wd = torch.from_numpy(W).cuda()
    w = qn.nf4_quantize(Wd)
    torch.cuda.synchronize()
    del Wd
    codes, q8, step = nf4_host(w)
    oc, oq, os_ = nf4.quantize(W)
    assert np.array_equal(codes, oc), f"{tag}: codes differ at bytes {np.nonzero(codes != oc)[0][:8]}"
    assert np.array_equal(q8, oq), f"{tag}: q8 differ at blocks {np.nonzero(q8 != oq)[0][:8]}"
    assert np.array_equal(step.view(np.uint32), os_.view(np.uint32)), f"{tag}: steps differ"
    say(f"[fullsize] {tag}: dequantize")
    deq = host_u16(qn.nf4_dequantize(w))
    torch.cuda.synchronize()
    od = nf4.dequantize(oc, oq, os_, N, K)
    assert np.array_equal(deq, od), f"{tag}: dequantized bits differ at {np.argwhere(deq != od)[:4]}"
    del deq, codes, oc
    return w, f32(od)


@pytest.mark.parametrize("wl,wi", _cases(fwd_only=False))
def test_fullsize_fwd_bwd(wl, wi):
    spec = wl.weights[wi]
    tag = f"{wl.name}/{spec.name}"
    inp = wl_mod.draw_workload_weight(wl, wi)
    M, N, K, r, s = inp.X.shape[0], spec.N, spec.K, wl.r, wl.s
    w, What = _quantize_and_check(inp.W, tag)

    say(f"[fullsize] {tag}: fwd + bwd M={M} r={r}")
    X, dY, A, B = dev_u16(inp.X), dev_u16(inp.dY), dev_u16(inp.A), dev_u16(inp.B)
    U = torch.empty(M, r, dtype=torch.bfloat16, device="cuda")
    Y = qn.qlora_linear_fwd(w, X, A, B, s, U_out=U)
    dX, dA, dB = qn.qlora_linear_bwd(w, X, dY, A, B, s, U=U)
    torch.cuda.synchronize()
    Yh, Uh, dXh, dAh, dBh = (f32(host_u16(t)) for t in (Y, U, dX, dA, dB))
    del X, dY, A, B, U, Y, dX, dA, dB, w
    torch.cuda.empty_cache()

    Xf, dYf, Af, Bf = f32(inp.X), f32(inp.dY), f32(inp.A), f32(inp.B)
    rows = _sample_rows(M, seed=1000 + wi)
    say(f"[fullsize] {tag}: oracle on {len(rows)} rows, adapters in full")
    e_u = assert_close("U", Uh, linear.lora_down(Xf, Af))
    e_y = assert_close("Y rows", Yh[rows], linear.forward_rows(Xf, What, Af, Bf, s, rows))
    e_dx = assert_close("dX rows", dXh[rows], linear.backward_rows(Xf, dYf, What, Af, Bf, s, rows))
    rA, rB = linear.adapter_grads(Xf, dYf, Af, Bf, s)
    e_da = assert_close("dA", dAh, rA)
    e_db = assert_close("dB", dBh, rB)
    say(f"[fullsize] {tag}: rel err U {e_u:.2e} Y {e_y:.2e} dX {e_dx:.2e} dA {e_da:.2e} dB {e_db:.2e}")


@pytest.mark.parametrize("wl,wi", _cases(fwd_only=True))
def test_fullsize_few_token_forward(wl, wi):
    spec = wl.weights[wi]
    tag = f"{wl.name}/{spec.name}"
    # the benchmark draws the largest token count and slices the others
    inp = wl_mod.draw_workload_weight(wl, wi, M=max(wl.M))
    N, K, r, s = spec.N, spec.K, wl.r, wl.s
    w, What = _quantize_and_check(inp.W, tag)
    A, B = dev_u16(inp.A), dev_u16(inp.B)
    Af, Bf = f32(inp.A), f32(inp.B)
    for M in wl.M:
        say(f"[fullsize] {tag}: forward M={M}")
        X = dev_u16(inp.X[:M])
        Y = qn.qlora_linear_fwd(w, X, A, B, s)
        torch.cuda.synchronize()
        Yh = f32(host_u16(Y))
        ref = linear.forward(f32(inp.X[:M]), What, Af, Bf, s)
        e = assert_close(f"Y M={M}", Yh, ref)
        say(f"[fullsize] {tag}: M={M} rel err Y {e:.2e}")
