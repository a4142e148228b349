"""Writes the golden fixtures in this folder.  Calls only the CPU oracle.

    python tests/golden/make_golden.py

nf4_levels_fp32.txt: the fp32 bit patterns of the 16 NF4 levels, defined as
normal quantiles with an exact zero, normalized to [-1, 1] ("QLoRA: fine-tuning
a 65B model on one GPU", section "NormalFloat, double quantization, paged
optimizers").

nf4_tiny_2x128.txt: a 2x128 weight of hand-picked fp32 values, its packed
codes, 8-bit constants, fp32 step and dequantized bf16 bits.
"""

import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import nf4  # noqa: E402


def tiny_weight():
    # deterministic, no random generator: a ramp, a sine and a few extremes
    i = np.arange(256, dtype=np.float64)
    w = 0.02 * np.sin(0.37 * i) * (1 + (i % 7 == 0) * 4)
    w[3] = 0.0
    w[130] = -0.25
    return w.astype(np.float32).reshape(2, 128)


def main():
    lv = nf4.nf4_levels().view(np.uint32)
    with open(os.path.join(HERE, "nf4_levels_fp32.txt"), "w") as f:
        f.write("# fp32 bits of the 16 NF4 levels, ascending (written by make_golden.py)\n")
        f.write(" ".join("%08x" % v for v in lv) + "\n")
    W = tiny_weight()
    packed, q8, step = nf4.quantize(W)
    deq = nf4.dequantize(packed, q8, step, 2, 128)
    with open(os.path.join(HERE, "nf4_tiny_2x128.txt"), "w") as f:
        f.write("# 2x128 weight (fp32 bits), codes, q8, step bits, dequantized bf16 bits\n")
        f.write("W " + " ".join("%08x" % v for v in W.view(np.uint32).reshape(-1)) + "\n")
        f.write("codes " + packed.tobytes().hex() + "\n")
        f.write("q8 " + q8.tobytes().hex() + "\n")
        f.write("step " + " ".join("%08x" % v for v in step.view(np.uint32)) + "\n")
        f.write("deq " + " ".join("%04x" % v for v in deq.reshape(-1)) + "\n")


if __name__ == "__main__":
    main()
