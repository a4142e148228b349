"""Helpers shared by the GPU parity tests: moving seeded host inputs to the
device, calling the C ABI through the thin binding, and the tolerance rule."""

import sys

import numpy as np
import torch

import quantized_base_lora_nf4_amd as qn
from oracle import linear, nf4

# Per tensor, against the fp64 oracle on the same bf16 inputs (bf16 inputs,
# fp32 accumulation, bf16 outputs):
#   max |gpu - ref| / max |ref|          <= TOL       (the layer's tolerance)
#   ||gpu - ref||_F / ||ref||_F          <= FROB_TOL  (a second, tighter gate:
#     bf16 rounding of the outputs and of U / dU gives about 1e-3, so a
#     dropped contraction block or a wrong adapter column, which can hide
#     under the max-norm gate, shows here)
TOL = 2e-2
FROB_TOL = 5e-3


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def dev_u16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def host_u16(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def f32(b: np.ndarray) -> np.ndarray:
    return nf4.bf16_bits_to_f32(b)


def gpu_quantize(W: np.ndarray, code: str = "nf4", blocksize: int = 64):
    Wd = torch.from_numpy(np.ascontiguousarray(W, dtype=np.float32)).cuda()
    w = qn.nf4_quantize(Wd, code=code, blocksize=blocksize)
    torch.cuda.synchronize()
    return w


def nf4_host(w):
    return (w.codes.cpu().numpy(), w.q8.cpu().numpy(), w.step.cpu().numpy())


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    ref = np.asarray(ref, np.float64)
    den = np.max(np.abs(ref))
    if den == 0:
        return float(np.max(np.abs(got)))
    return float(np.max(np.abs(np.asarray(got, np.float64) - ref)) / den)


def frob_err(got: np.ndarray, ref: np.ndarray) -> float:
    ref = np.asarray(ref, np.float64)
    d = np.asarray(got, np.float64) - ref
    den = float(np.sqrt(np.sum(ref * ref)))
    num = float(np.sqrt(np.sum(d * d)))
    return num if den == 0 else num / den


def assert_close(name: str, got: np.ndarray, ref: np.ndarray, tol: float = TOL,
                 frob_tol: float = FROB_TOL) -> float:
    """Both gates; prints both errors; returns the max-norm one."""
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    e = rel_err(got, ref)
    f = frob_err(got, ref)
    say(f"    {name}: max|d|/max|ref| = {e:.3e}  ||d||_F/||ref||_F = {f:.3e}")
    assert e <= tol, f"{name}: max|d|/max|ref| = {e:.3e} > {tol}"
    assert f <= frob_tol, f"{name}: ||d||_F/||ref||_F = {f:.3e} > {frob_tol}"
    return e


def oracle_what(W: np.ndarray, code: str = "nf4", blocksize: int = 64) -> np.ndarray:
    """Oracle-side quantize + dequantize, as fp32 values of the bf16 W_hat."""
    packed, q8, step = nf4.quantize(W, blocksize=blocksize, code=code)
    return f32(nf4.dequantize(packed, q8, step, *W.shape, blocksize=blocksize, code=code))
