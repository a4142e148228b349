"""Helpers shared by the GPU parity tests: moving seeded host inputs to the
device, calling the C ABI through the thin binding, and the tolerance rule."""

import sys

import numpy as np
import torch

import quantized_base_lora_nf4_amd as qn
from oracle import linear, nf4

# max |gpu - ref| / max |ref| per tensor (bf16 inputs, fp32 accumulation,
# fp64 reference)
TOL = 2e-2


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def dev_u16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def host_u16(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def f32(b: np.ndarray) -> np.ndarray:
    return nf4.bf16_bits_to_f32(b)


def gpu_quantize(W: np.ndarray, code: str = "nf4"):
    Wd = torch.from_numpy(np.ascontiguousarray(W, dtype=np.float32)).cuda()
    w = qn.nf4_quantize(Wd, code=code)
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


def assert_close(name: str, got: np.ndarray, ref: np.ndarray, tol: float = TOL) -> float:
    e = rel_err(got, ref)
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    assert e <= tol, f"{name}: max|d|/max|ref| = {e:.3e} > {tol}"
    return e


def oracle_what(W: np.ndarray, code: str = "nf4") -> np.ndarray:
    """Oracle-side quantize + dequantize, as fp32 values of the bf16 W_hat."""
    packed, q8, step = nf4.quantize(W, code=code)
    return f32(nf4.dequantize(packed, q8, step, *W.shape, code=code))


def oracle_what_from_state(codes, q8, step, N, K) -> np.ndarray:
    return f32(nf4.dequantize(codes, q8, step, N, K))
