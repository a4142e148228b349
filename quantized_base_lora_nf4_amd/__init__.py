"""Frozen-NF4-base + LoRA linear layer for AMD Instinct MI355X (gfx950).

The compute path is the HIP library ``libqlora_nf4.so`` behind the C ABI in
``include/qlora_nf4.h``; this package only loads it and marshals torch
tensors into its calls (see :mod:`quantized_base_lora_nf4_amd.ops`).
"""

from ._lib import LIB_PATH, EXPORTS, QloraError, lib  # noqa: F401
from .ops import (LqResult, NF4Weight, QLoRALinear, QLoRALinearFunction, alloc_nf4,  # noqa: F401
                  code_table, ilp_plan, lq_init, lq_workspace_size, nf4_dequantize,
                  nf4_quantize, qlora_linear_bwd, qlora_linear_fwd, qlora_linear_fwd_noalloc,
                  quant_error, storage_bytes, user_table, workspace_size, USER_CODES)
