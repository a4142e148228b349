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
                   QLORA_CODE_USER2, QLORA_CODE_USER3, QLORA_CODE_USER4, QLORA_ERR_INFEASIBLE,
                   Nf4Tensor, check, lib)

BLOCKSIZE = 64
DQ_BLOCKSIZE = 256
CODE_TYPES = {"nf4": QLORA_CODE_NF4, "fp4": QLORA_CODE_FP4, "nf3": QLORA_CODE_NF3,
              "nf2": QLORA_CODE_NF2, "user4": QLORA_CODE_USER4, "user3": QLORA_CODE_USER3,
              "user2": QLORA_CODE_USER2}
CODE_BITS = {"nf4": 4, "fp4": 4, "nf3": 3, "nf2": 2, "user4": 4, "user3": 3, "user2": 2}
# code types whose values the caller supplies (a codebook of 2^bits values)
USER_CODES = ("user4", "user3", "user2")


def _code_id(code: str) -> int:
    try:
        return CODE_TYPES[code]
    except KeyError:
        raise ValueError(f"code must be one of {sorted(CODE_TYPES)}, got {code!r}") from None


def _levels_array(code: str, levels) -> "ctypes.Array":
    """Host fp32 copy of a caller's codebook (2^bits values in code order)."""
    if levels is None:
        raise ValueError(f"code type {code!r} needs its 2^{CODE_BITS[code]} values (levels=)")
    vals = [float(v) for v in (levels.tolist() if hasattr(levels, "tolist") else levels)]
    if len(vals) != 2 ** CODE_BITS[code]:
        raise ValueError(f"{code!r} takes {2 ** CODE_BITS[code]} values, got {len(vals)}")
    arr = (ctypes.c_float * 16)()
    for i, v in enumerate(vals):
        arr[i] = v
    return arr


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
    code: str = "nf4"     # the code table: "nf4", "fp4", "nf3", "nf2" or "user4/3/2"
    blocksize: int = BLOCKSIZE  # elements per 8-bit constant: 64, 128 or 256
    levels: Optional[object] = None  # user code types: the codebook (2^bits values, host)

    def struct(self) -> Nf4Tensor:
        if self.levels is not None and not isinstance(self.levels, ctypes.Array):
            self.levels = _levels_array(self.code, self.levels)  # kept alive on self
        lv = ctypes.cast(self.levels, ctypes.c_void_p).value if self.levels is not None else None
        return Nf4Tensor(_ptr(self.codes), _ptr(self.q8), _ptr(self.step), self.N, self.K,
                         self.blocksize, DQ_BLOCKSIZE, _code_id(self.code), lv)

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


def user_table(code: str, levels) -> list:
    """The decision thresholds the library derives from a caller's codebook
    (code "user4", "user3" or "user2"); raises if the values break the
    contract (finite, |v| <= 1, and 0 or |v| >= 2^-20)."""
    arr = _levels_array(code, levels)
    th = (ctypes.c_float * 15)()
    n = lib().qlora_user_table(_code_id(code), ctypes.cast(arr, ctypes.c_void_p),
                               ctypes.cast(th, ctypes.c_void_p))
    check(min(n, 0), "qlora_user_table")
    return list(th)[:n]


BLOCKSIZES = (64, 128, 256)


def storage_bytes(N: int, K: int, code: str = "nf4", blocksize: int = BLOCKSIZE) -> int:
    """Bytes of the quantized state of one configuration (0 if unsupported)."""
    return int(lib().qlora_config_bytes(_code_id(code), blocksize, N, K))


def alloc_nf4(N: int, K: int, device="cuda", code: str = "nf4",
              blocksize: int = BLOCKSIZE) -> NF4Weight:
    if blocksize not in BLOCKSIZES or K % blocksize:
        raise ValueError(f"block size must be one of {BLOCKSIZES} and divide K")
    nb = N * K // blocksize
    ng = (nb + DQ_BLOCKSIZE - 1) // DQ_BLOCKSIZE
    return NF4Weight(
        codes=torch.empty(N * K * CODE_BITS[code] // 8, dtype=torch.uint8, device=device),
        q8=torch.empty(nb, dtype=torch.uint8, device=device),
        step=torch.empty(ng, dtype=torch.float32, device=device),
        N=N, K=K, code=code, blocksize=blocksize)


def nf4_quantize(W: torch.Tensor, out: Optional[NF4Weight] = None, stream=None,
                 code: str = "nf4", blocksize: int = BLOCKSIZE, levels=None) -> NF4Weight:
    """Quantize an fp32 [N, K] device tensor to block codes (NF4 by default,
    or FP4, NF3, NF2, or a caller's codebook: code "user4"/"user3"/"user2"
    with its 2^bits values in code order as `levels`) with double-quantized
    constants, one per `blocksize` elements (64, 128 or 256)."""
    if W.dtype != torch.float32 or W.dim() != 2:
        raise TypeError("W must be a 2-D float32 tensor")
    N, K = W.shape
    cid = _code_id(code)
    if code in USER_CODES:
        arr = _levels_array(code, levels)
    elif levels is not None:
        raise ValueError(f"code type {code!r} has built-in values; levels= is for user codes")
    else:
        arr = None
    if not W.is_cuda:
        raise ValueError("W must be a device tensor")
    if not W.is_contiguous():
        raise ValueError("W must be contiguous")
    if blocksize not in BLOCKSIZES or K % blocksize:
        raise ValueError(f"block size must be one of {BLOCKSIZES} and divide K")
    if out is None:
        with torch.cuda.stream(_stream_obj(stream)):  # allocated where the kernel writes
            out = alloc_nf4(N, K, W.device, code, blocksize)
    else:
        nb = N * K // blocksize
        if (out.codes.numel() != N * K * CODE_BITS[code] // 8 or out.q8.numel() != nb or
                out.step.numel() != -(-nb // DQ_BLOCKSIZE)):
            raise ValueError("out was allocated for another shape, code width or block size")
        _check_tensors([("out.codes", out.codes, out.codes.shape, False),
                        ("out.q8", out.q8, out.q8.shape, False),
                        ("out.step", out.step, out.step.shape, False)], W.device)
        if (out.codes.dtype != torch.uint8 or out.q8.dtype != torch.uint8 or
                out.step.dtype != torch.float32):
            raise TypeError("out: codes and q8 must be uint8, step float32")
        out.N, out.K, out.code, out.blocksize = N, K, code, blocksize
    out.levels = arr
    if arr is not None:
        st = lib().qlora_quantize_user(_ptr(W), N, K, cid, ctypes.cast(arr, ctypes.c_void_p),
                                       blocksize, DQ_BLOCKSIZE, _ptr(out.codes), _ptr(out.q8),
                                       _ptr(out.step), _stream(stream))
    elif cid == QLORA_CODE_NF4:
        st = lib().nf4_quantize(_ptr(W), N, K, blocksize, DQ_BLOCKSIZE, _ptr(out.codes),
                                _ptr(out.q8), _ptr(out.step), _stream(stream))
    else:
        st = lib().qlora_quantize(_ptr(W), N, K, cid, blocksize, DQ_BLOCKSIZE, _ptr(out.codes),
                                  _ptr(out.q8), _ptr(out.step), _stream(stream))
    check(st, "nf4_quantize")
    return out


def nf4_dequantize(w: NF4Weight, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Materialize the bf16 [N, K] weight (for checks and interop)."""
    dev = _check_weight(w)
    _check_tensors([("codes", w.codes, w.codes.shape, False), ("q8", w.q8, w.q8.shape, False),
                    ("step", w.step, w.step.shape, False), ("out", out, (w.N, w.K), True)], dev)
    if out is None:
        with torch.cuda.stream(_stream_obj(stream)):
            out = torch.empty(w.N, w.K, dtype=torch.bfloat16, device=dev)
    s = w.struct()
    check(lib().nf4_dequantize(ctypes.byref(s), _ptr(_bf16_view(out)), _stream(stream)),
          "nf4_dequantize")
    return out


def workspace_size(M: int, N: int, K: int, r: int, for_bwd: bool) -> int:
    return int(lib().qlora_workspace_size(M, N, K, r, 1 if for_bwd else 0))


def _stream_obj(stream):
    """The torch stream the kernels run on (a torch stream, a raw HIP stream
    handle, or None for the current stream)."""
    if stream is None:
        return torch.cuda.current_stream()
    if hasattr(stream, "cuda_stream"):
        return stream
    return torch.cuda.ExternalStream(int(stream))


def _check_tensors(items, device) -> None:
    """Shapes and dtypes, then devices and layout, of the tensors handed to a
    layer call: (name, tensor or None, expected shape, 16-bit?) tuples.  The
    C ABI sees bare pointers, so this is where a wrong shape or a tensor on
    another device is caught, before any launch."""
    for name, t, shape, sixteen in items:
        if t is None:
            continue
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch tensor")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        if sixteen and t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
            raise TypeError(f"{name} must be bf16 (or its 16-bit view), got {t.dtype}")
    for name, t, _, _ in items:
        if t is None:
            continue
        if not t.is_cuda or t.device != device:
            raise ValueError(f"{name} is on {t.device}, expected {device}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")


def _check_weight(w: NF4Weight) -> torch.device:
    if w.code not in CODE_TYPES:
        raise ValueError(f"unknown code type {w.code!r}")
    if w.codes.dtype != torch.uint8 or w.q8.dtype != torch.uint8 or w.step.dtype != torch.float32:
        raise TypeError("codes and q8 must be uint8, step float32")
    if w.codes.numel() != w.N * w.K * CODE_BITS[w.code] // 8:
        raise ValueError("codes do not match the weight's shape and code width")
    if w.code in USER_CODES and w.levels is None:
        raise ValueError(f"code type {w.code!r} needs its codebook (NF4Weight.levels)")
    if w.blocksize not in BLOCKSIZES:
        raise ValueError(f"block size must be one of {BLOCKSIZES}")
    if w.q8.numel() != w.N * w.K // w.blocksize or w.step.numel() != -(-w.q8.numel() // DQ_BLOCKSIZE):
        raise ValueError("q8 / step do not match the weight's shape")
    return w.codes.device


def _check_fwd(w: NF4Weight, X, A, B, Y, U_out, extra=()) -> Tuple[int, int, torch.device]:
    dev = _check_weight(w)
    if X.dim() != 2 or A.dim() != 2:
        raise ValueError("X and A must be 2-D")
    M, r = X.shape[0], A.shape[0]
    _check_tensors([("codes", w.codes, w.codes.shape, False), ("q8", w.q8, w.q8.shape, False),
                    ("step", w.step, w.step.shape, False),
                    ("X", X, (M, w.K), True), ("A", A, (r, w.K), True), ("B", B, (w.N, r), True),
                    ("Y", Y, (M, w.N), True), ("U", U_out, (M, r), True),
                    *[(n, t, shp(M, r), True) for n, t, shp in extra]], dev)
    return M, r, dev


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor]) -> torch.Tensor:
    if ws is not None:
        if not ws.is_cuda or ws.device != device or not ws.is_contiguous():
            raise ValueError("ws must be a contiguous tensor on the layer's GPU")
        if ws.numel() * ws.element_size() >= nbytes:
            return ws
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def qlora_linear_fwd(w: NF4Weight, X: torch.Tensor, A: torch.Tensor, B: torch.Tensor, s: float,
                     Y: Optional[torch.Tensor] = None, U_out: Optional[torch.Tensor] = None,
                     ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Y = X W^T + s (X A^T) B^T.  X [M, K], A [r, K], B [N, r] bf16.

    Buffers allocated here (Y, the workspace) are allocated on the stream the
    kernels run on, so the caching allocator does not hand them to other
    streams while those kernels may still use them."""
    M, r, dev = _check_fwd(w, X, A, B, Y, U_out)
    st = _stream_obj(stream)
    with torch.cuda.stream(st):
        if Y is None:
            Y = torch.empty(M, w.N, dtype=torch.bfloat16, device=dev)
        ws = _workspace(workspace_size(M, w.N, w.K, r, False), dev, ws)
    s_ = w.struct()
    rc = lib().qlora_linear_fwd(ctypes.byref(s_), _ptr(X), M, _ptr(A), _ptr(B), r, float(s),
                                _ptr(Y), _ptr(U_out), _ptr(ws), ws.numel() * ws.element_size(),
                                st.cuda_stream)
    check(rc, "qlora_linear_fwd")
    return Y


def qlora_linear_fwd_noalloc(w: NF4Weight, X: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
                             s: float, Y: torch.Tensor, U_out: Optional[torch.Tensor] = None,
                             stream=None) -> torch.Tensor:
    """qlora_linear_fwd without a workspace: the library's fixed device
    scratch is used and nothing is allocated (Y is the caller's)."""
    M, r, dev = _check_fwd(w, X, A, B, Y, U_out)
    s_ = w.struct()
    rc = lib().qlora_linear_fwd_noalloc(ctypes.byref(s_), _ptr(X), M, _ptr(A), _ptr(B), r,
                                        float(s), _ptr(Y), _ptr(U_out),
                                        _stream_obj(stream).cuda_stream)
    check(rc, "qlora_linear_fwd_noalloc")
    return Y


def qlora_linear_bwd(w: NF4Weight, X: torch.Tensor, dY: torch.Tensor, A: torch.Tensor,
                     B: torch.Tensor, s: float, U: Optional[torch.Tensor] = None,
                     need_dX: bool = True, out: Optional[tuple] = None,
                     ws: Optional[torch.Tensor] = None, stream=None):
    """Returns (dX or None, dA, dB), all bf16.  Buffers allocated here are
    allocated on the stream the kernels run on."""
    extra = [("dY", dY, lambda M, r: (M, w.N))]
    if out is not None:
        dX, dA, dB = out
        if dA is None or dB is None:
            raise ValueError("dA and dB outputs are required")
        extra += [("dX", dX, lambda M, r: (M, w.K)), ("dA", dA, lambda M, r: (r, w.K)),
                  ("dB", dB, lambda M, r: (w.N, r))]
    M, r, dev = _check_fwd(w, X, A, B, None, U, extra=extra)
    st = _stream_obj(stream)
    with torch.cuda.stream(st):
        if out is None:
            dX = torch.empty(M, w.K, dtype=torch.bfloat16, device=dev) if need_dX else None
            dA = torch.empty(r, w.K, dtype=torch.bfloat16, device=dev)
            dB = torch.empty(w.N, r, dtype=torch.bfloat16, device=dev)
        ws = _workspace(workspace_size(M, w.N, w.K, r, True), dev, ws)
    s_ = w.struct()
    rc = lib().qlora_linear_bwd(ctypes.byref(s_), _ptr(X), _ptr(dY), M, _ptr(A), _ptr(B), _ptr(U),
                                r, float(s), _ptr(dX), _ptr(dA), _ptr(dB), _ptr(ws),
                                ws.numel() * ws.element_size(), st.cuda_stream)
    check(rc, "qlora_linear_bwd")
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
                out: Optional[torch.Tensor] = None, stream=None,
                blocksize: int = BLOCKSIZE) -> torch.Tensor:
    """||R - W_hat(R)||_F^2 for one configuration (code type, block size),
    R = W or W - L1 L2t^T; returns a one-element float64 device tensor
    (written on the stream)."""
    if W.dtype != torch.float32 or W.dim() != 2:
        raise TypeError("W must be a 2-D float32 tensor")
    N, K = W.shape
    r = 0 if L1 is None else L1.shape[1]
    need = int(lib().qlora_config_error_workspace_size(N, K, _code_id(code), blocksize,
                                                       int(L1 is not None)))
    ws = _workspace(need, W.device, ws)
    if out is None:
        out = torch.empty(1, dtype=torch.float64, device=W.device)
    st = lib().qlora_config_error(_ptr(W), N, K, _code_id(code), blocksize, _ptr(L1), _ptr(L2t),
                                  r, _ptr(out), _ptr(ws), ws.numel() * ws.element_size(),
                                  _stream(stream))
    check(st, "qlora_config_error")
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
