"""Thin torch binding of the C ABI: argument marshalling only.

Tensors are torch CUDA (HIP) tensors; bf16 tensors may be ``torch.bfloat16``
or ``torch.int16``/``torch.uint16`` views of the bits.  Every call enqueues on
``torch.cuda.current_stream()`` unless a stream is passed.  All arithmetic
happens in the HIP kernels behind the C ABI.
"""

import ctypes
from dataclasses import dataclass
from typing import Optional, Tuple

import torch

from ._lib import (QLORA_CODE_FP4, QLORA_CODE_NF2, QLORA_CODE_NF3, QLORA_CODE_NF4,
                   QLORA_ERR_INFEASIBLE, Nf4Tensor, check, lib)

BLOCKSIZE = 64
DQ_BLOCKSIZE = 256
CODE_TYPES = {"nf4": QLORA_CODE_NF4, "fp4": QLORA_CODE_FP4, "nf3": QLORA_CODE_NF3,
              "nf2": QLORA_CODE_NF2}
CODE_BITS = {"nf4": 4, "fp4": 4, "nf3": 3, "nf2": 2}


def _code_id(code: str) -> int:
    try:
        return CODE_TYPES[code]
    except KeyError:
        raise ValueError(f"code must be one of {sorted(CODE_TYPES)}, got {code!r}") from None


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _bf16_view(t: torch.Tensor) -> torch.Tensor:
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return t
    raise TypeError(f"expected a bf16 tensor (or its 16-bit view), got {t.dtype}")


@dataclass
class NF4Weight:
    """Device storage of one quantized frozen weight."""
    codes: torch.Tensor   # uint8 [N*K*bits/8]
    q8: torch.Tensor      # uint8 [N*K/64]
    step: torch.Tensor    # float32 [ceil(N*K/16384)]
    N: int
    K: int
    code: str = "nf4"     # the code table the codes index: "nf4", "fp4", "nf3", "nf2"

    def struct(self) -> Nf4Tensor:
        return Nf4Tensor(_ptr(self.codes), _ptr(self.q8), _ptr(self.step), self.N, self.K,
                         BLOCKSIZE, DQ_BLOCKSIZE, _code_id(self.code))

    def nbytes(self) -> int:
        return self.codes.numel() + self.q8.numel() + 4 * self.step.numel()


def code_table(code: str = "nf4") -> Tuple[list, list]:
    """The library's code values (in code order, 2^bits of them) and its
    decision thresholds (15 for NF4, 14 for FP4, 7 for NF3, 3 for NF2), fp32."""
    lv = (ctypes.c_float * 16)()
    th = (ctypes.c_float * 15)()
    n = lib().qlora_code_table(_code_id(code), ctypes.cast(lv, ctypes.c_void_p),
                               ctypes.cast(th, ctypes.c_void_p))
    check(min(n, 0), "qlora_code_table")
    return list(lv)[:2 ** CODE_BITS[code]], list(th)[:n]


def storage_bytes(N: int, K: int, code: str = "nf4") -> int:
    return int(lib().qlora_storage_bytes(_code_id(code), N, K))


def alloc_nf4(N: int, K: int, device="cuda", code: str = "nf4") -> NF4Weight:
    nb = N * K // BLOCKSIZE
    ng = (nb + DQ_BLOCKSIZE - 1) // DQ_BLOCKSIZE
    return NF4Weight(
        codes=torch.empty(N * K * CODE_BITS[code] // 8, dtype=torch.uint8, device=device),
        q8=torch.empty(nb, dtype=torch.uint8, device=device),
        step=torch.empty(ng, dtype=torch.float32, device=device),
        N=N, K=K, code=code)


def nf4_quantize(W: torch.Tensor, out: Optional[NF4Weight] = None, stream=None,
                 code: str = "nf4") -> NF4Weight:
    """Quantize an fp32 [N, K] device tensor to block codes (NF4 by default,
    or FP4, NF3, NF2) with double-quantized constants."""
    if W.dtype != torch.float32 or W.dim() != 2:
        raise TypeError("W must be a 2-D float32 tensor")
    N, K = W.shape
    cid = _code_id(code)
    if out is None:
        out = alloc_nf4(N, K, W.device, code)
    elif out.codes.numel() != N * K * CODE_BITS[code] // 8:
        raise ValueError("out was allocated for another code width")
    else:
        out.code = code
    if cid == QLORA_CODE_NF4:
        st = lib().nf4_quantize(_ptr(W), N, K, BLOCKSIZE, DQ_BLOCKSIZE, _ptr(out.codes),
                                _ptr(out.q8), _ptr(out.step), _stream(stream))
    else:
        st = lib().qlora_quantize(_ptr(W), N, K, cid, BLOCKSIZE, DQ_BLOCKSIZE, _ptr(out.codes),
                                  _ptr(out.q8), _ptr(out.step), _stream(stream))
    check(st, "nf4_quantize")
    return out


def nf4_dequantize(w: NF4Weight, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Materialize the bf16 [N, K] weight (for checks and interop)."""
    if out is None:
        out = torch.empty(w.N, w.K, dtype=torch.bfloat16, device=w.codes.device)
    s = w.struct()
    check(lib().nf4_dequantize(ctypes.byref(s), _ptr(_bf16_view(out)), _stream(stream)),
          "nf4_dequantize")
    return out


def workspace_size(M: int, N: int, K: int, r: int, for_bwd: bool) -> int:
    return int(lib().qlora_workspace_size(M, N, K, r, 1 if for_bwd else 0))


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor]) -> torch.Tensor:
    if ws is not None and ws.numel() * ws.element_size() >= nbytes:
        return ws
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def qlora_linear_fwd(w: NF4Weight, X: torch.Tensor, A: torch.Tensor, B: torch.Tensor, s: float,
                     Y: Optional[torch.Tensor] = None, U_out: Optional[torch.Tensor] = None,
                     ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Y = X W^T + s (X A^T) B^T.  X [M, K], A [r, K], B [N, r] bf16."""
    M = X.shape[0]
    r = A.shape[0]
    if Y is None:
        Y = torch.empty(M, w.N, dtype=torch.bfloat16, device=X.device)
    nbytes = workspace_size(M, w.N, w.K, r, False)
    ws = _workspace(nbytes, X.device, ws)
    s_ = w.struct()
    st = lib().qlora_linear_fwd(ctypes.byref(s_), _ptr(_bf16_view(X)), M, _ptr(_bf16_view(A)),
                                _ptr(_bf16_view(B)), r, float(s), _ptr(_bf16_view(Y)),
                                _ptr(U_out), _ptr(ws), ws.numel() * ws.element_size(),
                                _stream(stream))
    check(st, "qlora_linear_fwd")
    return Y


def qlora_linear_bwd(w: NF4Weight, X: torch.Tensor, dY: torch.Tensor, A: torch.Tensor,
                     B: torch.Tensor, s: float, U: Optional[torch.Tensor] = None,
                     need_dX: bool = True, out: Optional[tuple] = None,
                     ws: Optional[torch.Tensor] = None, stream=None):
    """Returns (dX or None, dA, dB), all bf16."""
    M = X.shape[0]
    r = A.shape[0]
    dev = X.device
    if out is None:
        dX = torch.empty(M, w.K, dtype=torch.bfloat16, device=dev) if need_dX else None
        dA = torch.empty(r, w.K, dtype=torch.bfloat16, device=dev)
        dB = torch.empty(w.N, r, dtype=torch.bfloat16, device=dev)
    else:
        dX, dA, dB = out
    nbytes = workspace_size(M, w.N, w.K, r, True)
    ws = _workspace(nbytes, dev, ws)
    s_ = w.struct()
    st = lib().qlora_linear_bwd(ctypes.byref(s_), _ptr(_bf16_view(X)), _ptr(_bf16_view(dY)), M,
                                _ptr(_bf16_view(A)), _ptr(_bf16_view(B)), _ptr(U), r, float(s),
                                _ptr(dX), _ptr(dA), _ptr(dB), _ptr(ws),
                                ws.numel() * ws.element_size(), _stream(stream))
    check(st, "qlora_linear_bwd")
    return dX, dA, dB


LQ_START = {"svd": 0, "quantize": 1}


def lq_workspace_size(N: int, K: int, r: int, l: int) -> int:
    return int(lib().qlora_lq_workspace_size(N, K, r, l))


@dataclass
class LqResult:
    """Output of lq_init: the quantized part and the low-rank part."""
    w: NF4Weight
    A: torch.Tensor     # bf16 [r, K] = bf16(L2)
    B: torch.Tensor     # bf16 [N, r] = bf16(L1 / s)
    L1: torch.Tensor    # fp32 [N, r]
    L2t: torch.Tensor   # fp32 [K, r]


def lq_init(W: torch.Tensor, omega: torch.Tensor, r: int, iters: int = 2, power_iters: int = 2,
            start: str = "svd", s: float = 1.0, code: str = "nf4",
            ws: Optional[torch.Tensor] = None, stream=None) -> LqResult:
    """Split the fp32 [N, K] weight W into a quantized part and a rank-r part
    (alternating L and Q steps); omega is the fp32 [K, l] Gaussian test
    matrix of the randomized range finder."""
    if W.dtype != torch.float32 or W.dim() != 2 or omega.dtype != torch.float32:
        raise TypeError("W and omega must be float32, W 2-D")
    N, K = W.shape
    l = omega.shape[1]
    if omega.shape[0] != K:
        raise ValueError("omega must be [K, l]")
    dev = W.device
    w = alloc_nf4(N, K, dev, code)
    A = torch.empty(r, K, dtype=torch.bfloat16, device=dev)
    B = torch.empty(N, r, dtype=torch.bfloat16, device=dev)
    L1 = torch.empty(N, r, dtype=torch.float32, device=dev)
    L2t = torch.empty(K, r, dtype=torch.float32, device=dev)
    need = lq_workspace_size(N, K, r, l)
    ws = _workspace(need, dev, ws)
    st = lib().qlora_lq_init(_ptr(W), N, K, _code_id(code), r, l, _ptr(omega), iters, power_iters,
                             LQ_START[start], float(s), _ptr(w.codes), _ptr(w.q8), _ptr(w.step),
                             _ptr(A), _ptr(B), _ptr(L1), _ptr(L2t), _ptr(ws),
                             ws.numel() * ws.element_size(), _stream(stream))
    check(st, "qlora_lq_init")
    return LqResult(w=w, A=A, B=B, L1=L1, L2t=L2t)


def quant_error(W: torch.Tensor, code: str = "nf4", L1: Optional[torch.Tensor] = None,
                L2t: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """||R - W_hat(R)||_F^2 for one configuration, R = W or W - L1 L2t^T;
    returns a one-element float64 device tensor (written on the stream)."""
    if W.dtype != torch.float32 or W.dim() != 2:
        raise TypeError("W must be a 2-D float32 tensor")
    N, K = W.shape
    r = 0 if L1 is None else L1.shape[1]
    need = int(lib().qlora_quant_error_workspace_size(N, K, _code_id(code), int(L1 is not None)))
    ws = _workspace(need, W.device, ws)
    if out is None:
        out = torch.empty(1, dtype=torch.float64, device=W.device)
    st = lib().qlora_quant_error(_ptr(W), N, K, _code_id(code), _ptr(L1), _ptr(L2t), r,
                                 _ptr(out), _ptr(ws), ws.numel() * ws.element_size(),
                                 _stream(stream))
    check(st, "qlora_quant_error")
    return out


def ilp_plan(err, nbytes, budget: int):
    """Exact per-matrix configuration choice (host).  err, nbytes: [M][C]
    array-likes.  Returns (choice list, total error, total bytes), or None
    if nothing fits the budget."""
    import numpy as np
    e = np.ascontiguousarray(err, dtype=np.float64)
    b = np.ascontiguousarray(nbytes, dtype=np.int64)
    if e.ndim != 2 or e.shape != b.shape:
        raise ValueError("err and nbytes must be [M][C] arrays of the same shape")
    M, C = e.shape
    choice = np.zeros(M, dtype=np.int32)
    te = ctypes.c_double(0.0)
    tb = ctypes.c_int64(0)
    st = lib().qlora_ilp_plan(M, C, e.ctypes.data, b.ctypes.data, int(budget), choice.ctypes.data,
                              ctypes.byref(te), ctypes.byref(tb))
    if st == QLORA_ERR_INFEASIBLE:
        return None
    check(st, "qlora_ilp_plan")
    return [int(c) for c in choice], te.value, tb.value


class QLoRALinearFunction(torch.autograd.Function):
    """Autograd wrapper: gradients flow to X, A and B only (the NF4 base is frozen)."""

    @staticmethod
    def forward(ctx, X, A, B, w: NF4Weight, s: float):
        M = X.shape[0]
        U = torch.empty(M, A.shape[0], dtype=torch.bfloat16, device=X.device)
        Y = qlora_linear_fwd(w, X.contiguous(), A.contiguous(), B.contiguous(), s, U_out=U)
        ctx.save_for_backward(X, A, B, U)
        ctx.w = w
        ctx.s = s
        return Y

    @staticmethod
    def backward(ctx, dY):
        X, A, B, U = ctx.saved_tensors
        dX, dA, dB = qlora_linear_bwd(ctx.w, X.contiguous(), dY.contiguous(), A.contiguous(),
                                      B.contiguous(), ctx.s, U=U,
                                      need_dX=ctx.needs_input_grad[0])
        return dX, dA, dB, None, None


class QLoRALinear(torch.nn.Module):
    """A frozen NF4 weight with a trainable LoRA pair (A: r x K, B: N x r)."""

    def __init__(self, weight_fp32: torch.Tensor, r: int, alpha: float, A=None, B=None,
                 code: str = "nf4"):
        super().__init__()
        N, K = weight_fp32.shape
        self.nf4 = nf4_quantize(weight_fp32.float().contiguous(), code=code)
        self.r, self.alpha = r, alpha
        dev = weight_fp32.device
        self.A = torch.nn.Parameter(A if A is not None else
                                    (torch.randn(r, K, device=dev) * 0.01).bfloat16())
        self.B = torch.nn.Parameter(B if B is not None else
                                    torch.zeros(N, r, device=dev, dtype=torch.bfloat16))

    @property
    def s(self) -> float:
        return self.alpha / self.r

    def forward(self, X):
        shp = X.shape
        Y = QLoRALinearFunction.apply(X.reshape(-1, shp[-1]), self.A, self.B, self.nf4, self.s)
        return Y.reshape(*shp[:-1], Y.shape[-1])
