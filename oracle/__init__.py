"""CPU oracle for the frozen-NF4-base + LoRA linear layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call,
link or execute anything in this package: it exists so that tests, the
package's smoke check and the benchmark's CPU-baseline leg can check the HIP
path against a plain, slow, obviously correct restatement of what the layer
computes.  It shares no code, table or constant with the HIP library.

Sources (cited by page title and section):

* "QLoRA: fine-tuning a 65B model on one GPU" (blog post), sections
  "NormalFloat, double quantization, paged optimizers" and
  "Where the memory goes".
* "QLoRA: efficient finetuning of quantized LLMs" (CoChat paper page),
  Abstract.
* "ModuLoRA: Finetuning 2-Bit LLMs on Consumer GPUs by Integrating with
  Modular Quantizers" (paper record), abstract.
* "Qlora 4 Bit Quantization With Nf4 Fp4 Data Types And Lora Adapters"
  (capability page), entries on NF4 with double quantization.

Modules:

* :mod:`oracle.nf4` -- NF4 levels, blockwise absmax quantizer, double
  quantization, dequantization, bf16 round-to-nearest-even (numpy,
  vectorized).
* :mod:`oracle.scalar` -- the same quantizer as pure-Python scalar loops, for
  brute-force checks on tiny inputs.
* :mod:`oracle.linear` -- the layer's forward and backward in fp64.

Every function here is pinned by ``tests/test_oracle_*.py`` against facts
that do not come from the oracle itself (library routines, closed forms,
invariants, finite differences, brute force).  The one agreement that is not
pinned is between the NF4 level table derived here and any table published
outside the pages (the pages print no level values).
"""

from . import nf4, scalar, linear  # noqa: F401
