"""GPU parity of the configuration errors (qlora_quant_error) and of a
whole per-matrix plan under a memory budget, against the oracle (oracle.ilp).

* Without a low-rank part the dequantized weight is bit-exact, so the
  squared error differs only by summation order: relative 1e-12.
* With a low-rank part R = W - L1 L2t^T is formed in fp32 on the GPU and in
  fp64-then-fp32 by the oracle; an element can differ by one ulp and move a
  code at a near-tie: relative 1e-5.
* The plan from the GPU error table equals the oracle's plan from its own
  table (the planner itself is checked exactly against enumeration on the
  host).
"""

import numpy as np
import pytest
import torch

import quantized_base_lora_nf4_amd as qn
from oracle import ilp
from workloads import WeightSpec, draw_weight, rng_for
from gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    qn.lib()


def _gpu_err(W, code, L1=None, L2t=None, blocksize=64):
    Wd = torch.from_numpy(W).cuda()
    l1 = torch.from_numpy(L1).cuda() if L1 is not None else None
    l2 = torch.from_numpy(L2t).cuda() if L2t is not None else None
    out = qn.quant_error(Wd, code, l1, l2, blocksize=blocksize)
    torch.cuda.synchronize()
    return float(out.cpu().item())


SHAPES = [(1, 64), (7, 192), (300, 1024), (1024, 4160)]


@pytest.mark.parametrize("code", ilp.CODES)
@pytest.mark.parametrize("shape", SHAPES)
def test_quant_error_matches_oracle(code, shape):
    W = draw_weight(WeightSpec("w", *shape, 0.02, heavy_frac=0.01), rng_for(40, shape[0]))
    got = _gpu_err(W, code)
    want = ilp.quant_error(W, code)
    say(f"[ilp] {code} {shape}: {got:.10g} vs {want:.10g}")
    assert abs(got - want) <= 1e-12 * want


@pytest.mark.parametrize("code,bs", [("nf4", 64), ("nf2", 64), ("nf3", 256)])
def test_quant_error_with_low_rank_part(code, bs):
    N, K, r = 512, 1024, 16
    rng = rng_for(41, 0)
    W = draw_weight(WeightSpec("w", N, K, 0.02), rng)
    L1 = (rng.standard_normal((N, r)) * 0.02).astype(np.float32)
    L2t = (rng.standard_normal((K, r)) * 0.05).astype(np.float32)
    got = _gpu_err(W, code, L1, L2t, bs)
    want = ilp.quant_error(ilp.residual(W, L1, L2t), code, bs)
    say(f"[ilp] low rank {code}/{bs}: {got:.10g} vs {want:.10g}")
    assert abs(got - want) <= 1e-5 * want


def test_quant_error_of_zero_weight_is_zero():
    assert _gpu_err(np.zeros((16, 256), np.float32), "nf3") == 0.0


def test_plan_from_gpu_errors_matches_oracle():
    """Over every (code type, block size) configuration; four matrices keep
    the oracle's enumeration at 12^4 assignments."""
    specs = [WeightSpec("a", 256, 1024, 0.02), WeightSpec("b", 512, 512, 0.02, heavy_frac=0.01),
             WeightSpec("c", 128, 2048, 0.01), WeightSpec("d", 384, 768, 0.03, heavy_frac=0.02)]
    Ws = [draw_weight(sp, rng_for(42, i)) for i, sp in enumerate(specs)]
    err_g = np.array([[_gpu_err(W, c, blocksize=b) for c, b in ilp.CONFIGS] for W in Ws])
    err_o = np.array([[ilp.quant_error(W, c, b) for c, b in ilp.CONFIGS] for W in Ws])
    nbytes = np.array([[qn.storage_bytes(*W.shape, c, b) for c, b in ilp.CONFIGS] for W in Ws])
    assert np.array_equal(nbytes, [[ilp.state_bytes(*W.shape, c, b) for c, b in ilp.CONFIGS]
                                   for W in Ws])
    assert np.all(np.abs(err_g - err_o) <= 1e-12 * err_o)
    total_w = sum(W.size for W in Ws)
    for bits in (2.3, 2.6, 3.0, 3.6, 4.2, 4.6):
        budget = int(total_w * bits / 8)
        got = qn.ilp_plan(err_g, nbytes, budget)
        want = ilp.plan(err_o, nbytes, budget)
        say(f"[ilp] budget {bits} bits/weight: gpu {got and got[0]} oracle {want and list(want[0])}")
        if want is None:
            assert got is None
        else:
            assert list(want[0]) == got[0] and got[2] <= budget
