"""GPU parity of the low-rank plus quantized decomposition (qlora_lq_init)
against the fp64 oracle (oracle.lq), on the same W and test matrix Omega.

What must match and how:
* quantize-first, one iteration: Q is plain quantization of W, so codes,
  constants and steps are bit-exact;
* the low-rank part L1 L2t^T: max-norm-free relative Frobenius distance
  to the oracle's within 1e-3 where the spectrum has a gap (the planted
  inputs); where it has none (the quantization error of a Gaussian weight)
  the rank-r subspace is not unique, so the fit quality is compared
  instead: ||E - L|| within 0.2 % of the oracle's;
* Q after an L step quantizes W - L, which differs from the oracle's input
  by fp32 rounding: after one iteration codes may differ only at near-ties
  (at most 1e-4 of them), constants at most 2e-3 of them, steps by at most
  1e-5 relative (W - L is a few times smaller than L, so the fp32 rounding
  of L, about 4e-7 of it, is a few times larger relative to W - L).  A code decided differently at a near-tie changes that
  element of the next iteration's W - Q by a level gap, which moves the next
  L (by about 1e-4 relative) and with it more near-ties: from the second
  iteration on, at most 1e-3 of the codes, 2e-2 of the constants and 2e-3
  relative in the steps;
* the objective ||W - W_hat(Q) - L1 L2^T|| within 0.1 % of the oracle's;
* the adapter outputs are exactly bf16(L2) and bf16(fl32(L1 / s)) of the
  returned fp32 factors, and two runs are bit-identical.
"""

import numpy as np
import pytest
import torch

import quantized_base_lora_nf4_amd as qn
from oracle import lq, nf4
from workloads import draw_lq_inputs
from gpu_util import nf4_host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    qn.lib()


def _run(inp, iters, power_iters, start, code, s=0.25):
    W = torch.from_numpy(inp.W).cuda()
    Om = torch.from_numpy(inp.Omega).cuda()
    res = qn.lq_init(W, Om, inp.r, iters=iters, power_iters=power_iters, start=start, s=s,
                     code=code)
    torch.cuda.synchronize()
    return res


def _host(res):
    return (nf4_host(res.w), res.L1.cpu().numpy().astype(np.float64),
            res.L2t.cpu().numpy().astype(np.float64))


def _rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def _check_adapter(res, s):
    L1 = res.L1.cpu()
    L2t = res.L2t.cpu()
    A = res.A.cpu().view(torch.int16)
    B = res.B.cpu().view(torch.int16)
    assert torch.equal(A, L2t.t().contiguous().to(torch.bfloat16).view(torch.int16))
    assert torch.equal(B, (L1 / torch.tensor(s, dtype=torch.float32)).to(torch.bfloat16).view(torch.int16))


CASES = [  # N, K, r, l, iters, power_iters, start, code
    (300, 640, 12, 32, 1, 2, "svd", "nf4"),
    (300, 640, 12, 32, 2, 2, "svd", "nf4"),
    (173, 512, 8, 16, 2, 1, "svd", "nf3"),
    (1000, 1024, 16, 32, 3, 2, "svd", "nf4"),
    (512, 512, 40, 48, 1, 0, "svd", "nf2"),
    (256, 448, 88, 96, 1, 2, "svd", "nf4"),
    (300, 640, 12, 32, 2, 2, "quantize", "nf4"),
    (2048, 1024, 32, 48, 2, 2, "svd", "fp4"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "N%d_K%d_r%d_l%d_it%d_q%d_%s_%s" % c)
def test_lq_matches_oracle(case):
    N, K, r, l, iters, q, start, code = case
    say(f"[lq] {case}")
    inp = draw_lq_inputs(N, K, r, l, seed=7, index=N + K + r)
    res = _run(inp, iters, q, start, code)
    (codes, q8, step), L1, L2t = _host(res)
    (oc, oq, os_), oL1, oL2t = lq.decompose(inp.W, inp.Omega, r, iters, q, code=code, start=start)
    L, oL = L1 @ L2t.T, oL1 @ oL2t.T
    e_l = _rel(L, oL)
    obj = lq.objective(inp.W, (codes, q8, step), L1, L2t, code=code)
    oobj = lq.objective(inp.W, (oc, oq, os_), oL1, oL2t, code=code)
    cmis = np.mean(nf4.unpack_codes_k(codes, nf4.code_bits(code)) !=
                   nf4.unpack_codes_k(oc, nf4.code_bits(code)))
    qmis = np.mean(q8 != oq)
    srel = np.max(np.abs(step.astype(np.float64) - os_) / np.maximum(os_, 1e-30))
    say(f"[lq] L rel {e_l:.2e}  objective {obj:.6g} vs {oobj:.6g}  code mismatch {cmis:.1e}  "
        f"q8 mismatch {qmis:.1e}  step rel {srel:.1e}")
    if start == "quantize" and iters == 1:
        assert np.array_equal(codes, oc) and np.array_equal(q8, oq)
        assert np.array_equal(step.view(np.uint32), os_.view(np.uint32))
    if start == "svd":
        assert e_l <= 1e-3
    if iters == 1:
        assert cmis <= 1e-4 and qmis <= 2e-3 and srel <= 1e-5
    else:
        assert cmis <= 1e-3 and qmis <= 2e-2 and srel <= 2e-3
    assert abs(obj - oobj) <= 1e-3 * oobj
    _check_adapter(res, 0.25)


def test_quantize_first_fits_the_quantization_error():
    N, K, r, l = 400, 512, 16, 32
    inp = draw_lq_inputs(N, K, r, l, seed=8, strength=0.0)   # plain Gaussian weight
    res = _run(inp, 1, 2, "quantize", "nf4")
    (codes, q8, step), L1, L2t = _host(res)
    state = nf4.quantize(inp.W)
    assert np.array_equal(codes, state[0])
    E = lq.quant_error_f32(inp.W, state, "nf4").astype(np.float64)
    oL1, oL2t = lq.low_rank(E, inp.Omega, r, 2)
    fit = np.linalg.norm(E - L1 @ L2t.T)
    ofit = np.linalg.norm(E - oL1 @ oL2t.T)
    say(f"[lq] white error: fit {fit:.6g} vs oracle {ofit:.6g}")
    assert abs(fit - ofit) <= 2e-3 * ofit


def test_lq_is_deterministic():
    inp = draw_lq_inputs(300, 640, 12, 32, seed=9)
    a = _run(inp, 2, 2, "svd", "nf4")
    b = _run(inp, 2, 2, "svd", "nf4")
    for x, y in ((a.w.codes, b.w.codes), (a.w.q8, b.w.q8), (a.L1, b.L1), (a.L2t, b.L2t), (a.A, b.A)):
        assert torch.equal(x.view(torch.uint8) if x.dtype != torch.bfloat16 else x.view(torch.int16),
                           y.view(torch.uint8) if y.dtype != torch.bfloat16 else y.view(torch.int16))


def test_lq_full_size_q_proj():
    """The 4096 x 4096 projection of the LLaMA-7B workload at rank 64."""
    N = K = 4096
    r, l = 64, 80
    inp = draw_lq_inputs(N, K, r, l, seed=0, index=0)
    say("[lq] full size 4096x4096 r=64 l=80, 2 iterations")
    res = _run(inp, 2, 2, "svd", "nf4")
    (codes, q8, step), L1, L2t = _host(res)
    (oc, oq, os_), oL1, oL2t = lq.decompose(inp.W, inp.Omega, r, 2, 2)
    e_l = _rel(L1 @ L2t.T, oL1 @ oL2t.T)
    obj = lq.objective(inp.W, (codes, q8, step), L1, L2t)
    oobj = lq.objective(inp.W, (oc, oq, os_), oL1, oL2t)
    cmis = np.mean(nf4.unpack_codes(codes) != nf4.unpack_codes(oc))
    say(f"[lq] full size: L rel {e_l:.2e} objective {obj:.6g} vs {oobj:.6g} code mismatch {cmis:.1e}")
    assert e_l <= 1e-3 and abs(obj - oobj) <= 1e-3 * oobj and cmis <= 1e-3


def test_lq_rank_deficient_weight():
    """W of exact rank 4 (up to its fp32 rounding) with l = 32: the sampled
    range has 4 real directions, and the orthonormalization must drop the
    other 28.  The GPU drops a Cholesky pivot below 1e-10 of the largest
    diagonal of the Gram matrix, the oracle an eigenvalue below 1e-10 of the
    largest: different rules that must keep the same span here.  Both
    low-rank parts then reproduce W to fp32 rounding, and W - L is rounding
    noise, so the codes of Q are not compared; the objective is (about 1e-6
    of ||W||)."""
    N, K, r, l = 300, 640, 12, 32
    rng = np.random.default_rng(21)
    W = ((rng.standard_normal((N, 4)) @ rng.standard_normal((4, K))) * 0.01).astype(np.float32)
    Om = rng.standard_normal((K, l)).astype(np.float32)

    class Inp:
        pass
    inp = Inp()
    inp.W, inp.Omega, inp.r, inp.l = W, Om, r, l
    res = _run(inp, 1, 2, "svd", "nf4")
    (codes, q8, step), L1, L2t = _host(res)
    assert np.all(np.isfinite(L1)) and np.all(np.isfinite(L2t))
    (oc, oq, os_), oL1, oL2t = lq.decompose(W, Om, r, 1, 2)
    L, oL = L1 @ L2t.T, oL1 @ oL2t.T
    Wd = W.astype(np.float64)
    say(f"[lq] rank 4: |L-W|/|W| {_rel(L, Wd):.2e}  |oL-W|/|W| {_rel(oL, Wd):.2e}  "
        f"|L-oL|/|oL| {_rel(L, oL):.2e}")
    assert _rel(oL, Wd) <= 1e-6
    assert _rel(L, Wd) <= 1e-5 and _rel(L, oL) <= 1e-5
    obj = lq.objective(W, (codes, q8, step), L1, L2t)
    assert obj <= 1e-5 * np.linalg.norm(Wd)
    _check_adapter(res, 0.25)
