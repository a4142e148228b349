"""ctypes loader for libqlora_nf4.so and the raw C signatures.

The library is built in place by ``quantized_base_lora_nf4_amd.build``.  If
it is missing, every entry point raises: there is no CPU fallback.
"""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqlora_nf4.so")

QLORA_OK = 0
QLORA_ERR_INVALID = -1
QLORA_ERR_UNSUPPORTED = -2
QLORA_ERR_WORKSPACE = -3
QLORA_ERR_LAUNCH = -4
QLORA_ERR_INFEASIBLE = -5

QLORA_CODE_NF4 = 0
QLORA_CODE_FP4 = 1
QLORA_CODE_NF3 = 2
QLORA_CODE_NF2 = 3
QLORA_CODE_USER4 = 4
QLORA_CODE_USER3 = 5
QLORA_CODE_USER2 = 6
QLORA_USER_MIN_MAGNITUDE = 2.0 ** -20

# Size of the fixed device scratch of qlora_linear_fwd_noalloc
QLORA_NOALLOC_SCRATCH_BYTES = 16 << 20
# Workgroups (and sink words) of qlora_stream_read
QLORA_STREAM_GRID = 1024

# Every symbol the header declares.
EXPORTS = (
    "qlora_status_str",
    "nf4_code_table",
    "qlora_code_table",
    "nf4_storage_bytes",
    "qlora_storage_bytes",
    "nf4_quantize",
    "qlora_quantize",
    "qlora_quantize_user",
    "qlora_user_table",
    "nf4_dequantize",
    "qlora_workspace_size",
    "qlora_linear_fwd",
    "qlora_linear_bwd",
    "qlora_linear_fwd_ev",
    "qlora_linear_bwd_ev",
    "qlora_linear_fwd_noalloc",
    "qlora_stream_read",
    "qlora_lq_workspace_size",
    "qlora_lq_init",
    "qlora_quant_error_workspace_size",
    "qlora_quant_error",
    "qlora_ilp_plan",
    "qlora_config_bytes",
    "qlora_config_error_workspace_size",
    "qlora_config_error",
)


class Nf4Tensor(ctypes.Structure):
    """Mirror of nf4_tensor_t."""
    _fields_ = [
        ("codes", ctypes.c_void_p),
        ("q8", ctypes.c_void_p),
        ("step", ctypes.c_void_p),
        ("N", ctypes.c_int64),
        ("K", ctypes.c_int64),
        ("blocksize", ctypes.c_int32),
        ("dq_blocksize", ctypes.c_int32),
        ("code_type", ctypes.c_int32),
        ("levels", ctypes.c_void_p),
    ]


class QloraError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: status {status} ({status_str(status)})")


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"HIP library not built: {LIB_PATH} is missing. "
            "Run `python -m quantized_base_lora_nf4_amd.build` (hipcc, gfx950).")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, f32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    L.qlora_status_str.restype = ctypes.c_char_p
    L.qlora_status_str.argtypes = [i32]
    L.nf4_code_table.restype = None
    L.nf4_code_table.argtypes = [vp, vp]
    L.qlora_code_table.restype = i32
    L.qlora_code_table.argtypes = [i32, vp, vp]
    L.nf4_storage_bytes.restype = sz
    L.nf4_storage_bytes.argtypes = [i64, i64]
    L.qlora_storage_bytes.restype = sz
    L.qlora_storage_bytes.argtypes = [i32, i64, i64]
    L.nf4_quantize.restype = i32
    L.nf4_quantize.argtypes = [vp, i64, i64, i32, i32, vp, vp, vp, vp]
    L.qlora_quantize.restype = i32
    L.qlora_quantize.argtypes = [vp, i64, i64, i32, i32, i32, vp, vp, vp, vp]
    L.qlora_quantize_user.restype = i32
    L.qlora_quantize_user.argtypes = [vp, i64, i64, i32, vp, i32, i32, vp, vp, vp, vp]
    L.qlora_user_table.restype = i32
    L.qlora_user_table.argtypes = [i32, vp, vp]
    L.nf4_dequantize.restype = i32
    L.nf4_dequantize.argtypes = [ctypes.POINTER(Nf4Tensor), vp, vp]
    L.qlora_workspace_size.restype = sz
    L.qlora_workspace_size.argtypes = [i64, i64, i64, i32, i32]
    L.qlora_linear_fwd.restype = i32
    L.qlora_linear_fwd.argtypes = [ctypes.POINTER(Nf4Tensor), vp, i64, vp, vp, i32, f32, vp, vp,
                                   vp, sz, vp]
    L.qlora_linear_bwd.restype = i32
    L.qlora_linear_bwd.argtypes = [ctypes.POINTER(Nf4Tensor), vp, vp, i64, vp, vp, vp, i32, f32,
                                   vp, vp, vp, vp, sz, vp]
    L.qlora_linear_fwd_ev.restype = i32
    L.qlora_linear_fwd_ev.argtypes = L.qlora_linear_fwd.argtypes + [vp, vp]
    L.qlora_linear_bwd_ev.restype = i32
    L.qlora_linear_bwd_ev.argtypes = L.qlora_linear_bwd.argtypes + [vp, vp]
    L.qlora_linear_fwd_noalloc.restype = i32
    L.qlora_linear_fwd_noalloc.argtypes = [ctypes.POINTER(Nf4Tensor), vp, i64, vp, vp, i32, f32,
                                           vp, vp, vp]
    L.qlora_stream_read.restype = i32
    L.qlora_stream_read.argtypes = [vp, sz, vp, vp]
    L.qlora_lq_workspace_size.restype = sz
    L.qlora_lq_workspace_size.argtypes = [i64, i64, i32, i32]
    L.qlora_lq_init.restype = i32
    L.qlora_lq_init.argtypes = [vp, i64, i64, i32, i32, i32, vp, i32, i32, i32, f32,
                                vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.qlora_quant_error_workspace_size.restype = sz
    L.qlora_quant_error_workspace_size.argtypes = [i64, i64, i32, i32]
    L.qlora_quant_error.restype = i32
    L.qlora_quant_error.argtypes = [vp, i64, i64, i32, vp, vp, i32, vp, vp, sz, vp]
    L.qlora_config_bytes.restype = sz
    L.qlora_config_bytes.argtypes = [i32, i32, i64, i64]
    L.qlora_config_error_workspace_size.restype = sz
    L.qlora_config_error_workspace_size.argtypes = [i64, i64, i32, i32, i32]
    L.qlora_config_error.restype = i32
    L.qlora_config_error.argtypes = [vp, i64, i64, i32, i32, vp, vp, i32, vp, vp, sz, vp]
    L.qlora_ilp_plan.restype = i32
    L.qlora_ilp_plan.argtypes = [i32, i32, vp, vp, i64, vp, vp, vp]
    _lib = L
    return L


def status_str(status: int) -> str:
    try:
        return lib().qlora_status_str(int(status)).decode()
    except RuntimeError:
        return "library not loaded"


def check(status: int, what: str) -> None:
    if status != QLORA_OK:
        raise QloraError(status, what)
