"""Seeded synthetic inputs and workload shapes for the NF4 + LoRA linear layer.

This module only draws random numbers and names shapes.  It holds none of
the layer's arithmetic (no quantization, no dequantization, no products), so
that both the CPU oracle and the HIP path can be fed the same bytes.

Draw order per weight: W (fp32) -> heavy-tail mask (if any) -> X -> dY ->
A -> B, from numpy's PCG64 seeded with the SeedSequence (seed, weight index).
Every bf16 tensor is drawn in fp32 and rounded to bf16 by torch's CPU cast
(round to nearest even); it is handed over as uint16 bit patterns.

The shapes stand in for the projection layers of LLaMA-7B, -13B and -65B
class models; no weights or datasets are used.
"""

from dataclasses import dataclass
from typing import Optional, Tuple

import numpy as np
import torch


@dataclass(frozen=True)
class WeightSpec:
    name: str
    N: int
    K: int
    sigma: float
    heavy_frac: float = 0.0     # fraction of entries scaled by heavy_mult
    heavy_mult: float = 10.0


@dataclass(frozen=True)
class Workload:
    name: str
    weights: Tuple[WeightSpec, ...]
    M: Tuple[int, ...]          # token counts (several only for the GEMV case)
    r: int
    alpha: float
    fwd_only: bool = False
    ab_sigma: float = 0.01
    seed: int = 0
    note: str = ""

    @property
    def s(self) -> float:
        return self.alpha / self.r


# The five workloads.  Names describe what they are.
SINGLE_1K = Workload(
    name="single_1024x1024_M256_r8",
    weights=(WeightSpec("w", 1024, 1024, 0.02),),
    M=(256,), r=8, alpha=16.0,
    note="one 1024x1024 weight, 256 tokens, LoRA r=8 alpha=16",
)
LLAMA7B_QUP = Workload(
    name="llama7b_q_up_M4096_r64",
    weights=(WeightSpec("q_proj", 4096, 4096, 0.02, heavy_frac=0.01),
             WeightSpec("up_proj", 11008, 4096, 0.02, heavy_frac=0.01)),
    M=(4096,), r=64, alpha=16.0,
    note="LLaMA-7B q_proj and up_proj shapes, 1% of entries x10, 4096 tokens (8 x 512)",
)
LLAMA65B_MLP = Workload(
    name="llama65b_mlp_M4096_r64",
    weights=(WeightSpec("gate_proj", 22016, 8192, 0.015),
             WeightSpec("up_proj", 22016, 8192, 0.015),
             WeightSpec("down_proj", 8192, 22016, 0.015)),
    M=(4096,), r=64, alpha=16.0,
    note="LLaMA-65B MLP shapes, 4096 tokens",
)
SKINNY_GEMV = Workload(
    name="skinny_gemv_8192_28672x8192_M1_4_16_r16",
    weights=(WeightSpec("w8k", 8192, 8192, 0.02),
             WeightSpec("w28k", 28672, 8192, 0.02)),
    M=(1, 4, 16), r=16, alpha=32.0, fwd_only=True,
    note="bandwidth-bound forward for 1, 4 and 16 tokens",
)
LLAMA13B_BLOCK = Workload(
    name="llama13b_block_M2048_r64",
    weights=(WeightSpec("q_proj", 5120, 5120, 0.02),
             WeightSpec("k_proj", 5120, 5120, 0.02),
             WeightSpec("v_proj", 5120, 5120, 0.02),
             WeightSpec("o_proj", 5120, 5120, 0.02),
             WeightSpec("gate_proj", 13824, 5120, 0.02),
             WeightSpec("up_proj", 13824, 5120, 0.02),
             WeightSpec("down_proj", 5120, 13824, 0.02)),
    M=(2048,), r=64, alpha=16.0,
    note="LLaMA-13B decoder block projections, 2048 tokens, quantize included",
)

WORKLOADS = (SINGLE_1K, LLAMA7B_QUP, LLAMA65B_MLP, SKINNY_GEMV, LLAMA13B_BLOCK)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16) via torch's CPU cast."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_float(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 values via torch's CPU cast."""
    t = torch.from_numpy(np.ascontiguousarray(b, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(torch.float32).numpy().copy()


def rng_for(seed: int, index: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, index])))


def draw_weight(spec: WeightSpec, rng: np.random.Generator) -> np.ndarray:
    """W [N, K] fp32 ~ N(0, sigma^2); if heavy_frac > 0, an i.i.d.
    Bernoulli(heavy_frac) mask picks entries that are multiplied by
    heavy_mult."""
    W = rng.standard_normal((spec.N, spec.K), dtype=np.float32)
    W *= np.float32(spec.sigma)
    if spec.heavy_frac > 0:
        mask = rng.random((spec.N, spec.K), dtype=np.float32) < spec.heavy_frac
        W[mask] *= np.float32(spec.heavy_mult)
    return W


@dataclass
class LayerInputs:
    """One weight's inputs.  bf16 tensors are uint16 bit patterns."""
    W: np.ndarray                 # fp32 [N, K]
    X: np.ndarray                 # bf16 [M, K]
    dY: Optional[np.ndarray]      # bf16 [M, N] (None for forward-only)
    A: np.ndarray                 # bf16 [r, K]
    B: np.ndarray                 # bf16 [N, r]
    s: float
    r: int


def draw_layer(N: int, K: int, M: int, r: int, s: float, *, sigma: float = 0.02,
               heavy_frac: float = 0.0, ab_sigma: float = 0.01, seed: int = 0,
               index: int = 0, with_dy: bool = True) -> LayerInputs:
    rng = rng_for(seed, index)
    W = draw_weight(WeightSpec("w", N, K, sigma, heavy_frac), rng)
    X = to_bf16_bits(rng.standard_normal((M, K), dtype=np.float32))
    dY = to_bf16_bits(rng.standard_normal((M, N), dtype=np.float32)) if with_dy else None
    A = to_bf16_bits(rng.standard_normal((r, K), dtype=np.float32) * np.float32(ab_sigma))
    B = to_bf16_bits(rng.standard_normal((N, r), dtype=np.float32) * np.float32(ab_sigma))
    return LayerInputs(W=W, X=X, dY=dY, A=A, B=B, s=s, r=r)


def draw_workload_weight(wl: Workload, wi: int, M: Optional[int] = None) -> LayerInputs:
    spec = wl.weights[wi]
    return draw_layer(spec.N, spec.K, M if M is not None else wl.M[0], wl.r, wl.s,
                      sigma=spec.sigma, heavy_frac=spec.heavy_frac, ab_sigma=wl.ab_sigma,
                      seed=wl.seed, index=wi, with_dy=not wl.fwd_only)


@dataclass
class LqInputs:
    """Inputs of the low-rank plus quantized decomposition of one weight."""
    W: np.ndarray       # fp32 [N, K]
    Omega: np.ndarray   # fp32 [K, l], the random test matrix of the range finder
    r: int
    l: int


def draw_lq_inputs(N: int, K: int, r: int, l: int, *, sigma: float = 0.02, rank0: Optional[int] = None,
                   strength: float = 3.0, seed: int = 0, index: int = 0) -> LqInputs:
    """W = sigma (G + P): G [N, K] i.i.d. N(0, 1), plus a planted component
    P = strength (sqrt N + sqrt K) U0 V0^T of rank rank0 (default r), with
    U0 [N, rank0] and V0 [K, rank0] i.i.d. N(0, 1) scaled by 1/sqrt(N) and
    1/sqrt(K).  The planted singular values sit near strength times the edge
    sqrt N + sqrt K of G's spectrum, which gives a pretrained-like matrix a
    few dominant directions and a clear gap after them.  Omega [K, l] is
    i.i.d. N(0, 1).  Draw order: G, U0, V0, Omega."""
    rank0 = r if rank0 is None else rank0
    rng = rng_for(seed, 1000 + index)
    G = rng.standard_normal((N, K), dtype=np.float32)
    U0 = rng.standard_normal((N, rank0)) / np.sqrt(N)
    V0 = rng.standard_normal((K, rank0)) / np.sqrt(K)
    P = (strength * (np.sqrt(N) + np.sqrt(K))) * (U0 @ V0.T)
    W = (np.float64(sigma) * (G.astype(np.float64) + P)).astype(np.float32)
    Omega = rng.standard_normal((K, l), dtype=np.float32)
    return LqInputs(W=W, Omega=Omega, r=r, l=l)



CODEBOOK_KINDS = ("plain", "with_zero", "repeats", "symmetric", "clustered")


def draw_codebook(rng: np.random.Generator, bits: int, kind: str = "plain") -> np.ndarray:
    """A caller's codebook of 2^bits fp32 values in shuffled code order,
    within the contract (|v| <= 1, and 0 or |v| >= 2^-20):
      plain      uniform on [-1, 1]
      with_zero  one value exactly 0
      repeats    two pairs of equal values
      symmetric  no zero, every value mirrored (a midpoint at 0)
      clustered  values 1 ulp apart and their negatives
    """
    n = 2 ** bits
    v = rng.uniform(-1.0, 1.0, n).astype(np.float32)
    v[(v != 0) & (np.abs(v) < 2.0 ** -20)] = np.float32(2.0 ** -20)
    if kind == "with_zero":
        v[rng.integers(n)] = 0.0
    elif kind == "repeats":
        v[1] = v[0]
        v[-1] = v[-2]
    elif kind == "symmetric":
        h = np.abs(v[: n // 2]) + np.float32(2.0 ** -20)
        v = np.concatenate([-h, h]).astype(np.float32)
    elif kind == "clustered":
        base = np.float32(rng.uniform(0.1, 0.9))
        v = np.array([base] * n, np.float32)
        for i in range(1, n):
            v[i] = np.nextafter(v[i - 1], np.float32(2.0)) if i % 2 else -v[i - 1]
    elif kind != "plain":
        raise ValueError(kind)
    rng.shuffle(v)
    return v
