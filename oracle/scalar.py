"""Pure-Python scalar NF4 quantizer, for brute-force checks on tiny inputs.
Test infrastructure only.

It follows the same steps as :mod:`oracle.nf4` (blockwise absmax, divide,
nearest code value with ties to the lower value, pack, double quantization,
dequantization) one element at a time, with no numpy in the arithmetic.
Python floats are fp64; fp32 results are obtained by rounding the fp64 result
of one operation on fp32 operands to fp32.  For a single division or
multiplication of fp32 operands this gives the correctly rounded fp32 result
(fp64 carries more than 2*24 + 2 significand bits, so the two roundings
cannot disagree with one direct rounding).

Page citations are those of :mod:`oracle.nf4` ("QLoRA: fine-tuning a 65B
model on one GPU", section "NormalFloat, double quantization, paged
optimizers"; "Qlora 4 Bit Quantization With Nf4 Fp4 Data Types And Lora
Adapters", NF4 entry).
"""

import math
import struct


def f32(x: float) -> float:
    """Round a Python float to the nearest fp32 (ties to even)."""
    return struct.unpack("<f", struct.pack("<f", x))[0]


def f32_bits(x: float) -> int:
    return struct.unpack("<I", struct.pack("<f", x))[0]


def bf16_bits(x: float) -> int:
    """Round an fp32 value to bf16, ties to even, by comparing the two bf16
    neighbours of x directly (no bit tricks)."""
    b = f32_bits(x)
    lo = b & 0xFFFF0000
    hi = lo + 0x10000
    vlo = struct.unpack("<f", struct.pack("<I", lo))[0]
    if b == lo:
        return lo >> 16
    if (hi & 0x7F800000) == 0x7F800000 and (hi & 0x007FFFFF) == 0:
        # rounding past the largest finite bf16: IEEE compares against the
        # next value the format would have with an unbounded exponent, 2^128
        vhi = math.copysign(2.0 ** 128, vlo)
    else:
        vhi = struct.unpack("<f", struct.pack("<I", hi & 0xFFFFFFFF))[0]
    dlo = abs(x - vlo)
    dhi = abs(vhi - x)
    if dlo < dhi:
        return lo >> 16
    if dhi < dlo:
        return (hi >> 16) & 0xFFFF
    return (lo >> 16) if ((lo >> 16) & 1) == 0 else ((hi >> 16) & 0xFFFF)


def pack_kbit(codes, bits):
    """Pack a flat list of codes (length a multiple of 64) into bytes.

    bits = 4: element 2j in the low nibble of byte j.  bits = 3 or 2: per
    64-element block, 2 * bits little-endian 32-bit words; element
    e = 32 h + 8 g + 2 i + p puts code bits 0-1 at bit 8 i + 2 g of word
    bits * h + p and, for 3 bits, code bit 2 at bit (8 i + 2 + 2 g + p) % 32
    of word 3 h + 2.
    """
    if bits == 4:
        return bytes(codes[2 * j] | (codes[2 * j + 1] << 4) for j in range(len(codes) // 2))
    out = bytearray()
    for b0 in range(0, len(codes), 64):
        words = [0] * (2 * bits)
        for e in range(64):
            c = codes[b0 + e]
            h, g, i, p = e // 32, (e // 8) % 4, (e // 2) % 4, e % 2
            words[bits * h + p] |= (c & 3) << (8 * i + 2 * g)
            if bits == 3:
                words[3 * h + 2] |= ((c >> 2) & 1) << ((8 * i + 2 + 2 * g + p) % 32)
        for w in words:
            out += struct.pack("<I", w)
    return bytes(out)


def unpack_kbit(packed, bits, n):
    """Inverse of pack_kbit for n codes."""
    if bits == 4:
        out = []
        for byte in packed:
            out += [byte & 0xF, byte >> 4]
        return out[:n]
    out = []
    wb = 8 * bits  # bytes per block
    for b0 in range(0, n, 64):
        blk = packed[(b0 // 64) * wb:(b0 // 64 + 1) * wb]
        words = list(struct.unpack("<%dI" % (2 * bits), blk))
        for e in range(64):
            h, g, i, p = e // 32, (e // 8) % 4, (e // 2) % 4, e % 2
            c = (words[bits * h + p] >> (8 * i + 2 * g)) & 3
            if bits == 3:
                c |= ((words[3 * h + 2] >> ((8 * i + 2 + 2 * g + p) % 32)) & 1) << 2
            out.append(c)
    return out


def quantize(W, levels, blocksize=64, dq_blocksize=256):
    """W: list of rows (lists of fp32-representable floats).  levels: the 16
    fp32-representable code values in code order (ascending for NF4; for
    FP4 the E2M1 order, with +0 and -0).  Each element gets the code of the
    nearest value; a tie between two values goes to the lower value, and
    two codes with the same value to the lower code.  Returns (codes bytes,
    q8 list, step list)."""
    flat = [float(v) for row in W for v in row]
    n = len(flat)
    assert n % blocksize == 0
    nb = n // blocksize
    c = []
    codes = []
    for b in range(nb):
        blk = flat[b * blocksize:(b + 1) * blocksize]
        cb = 0.0
        for w in blk:
            if abs(w) > cb:
                cb = abs(w)
        c.append(cb)
        for w in blk:
            x = 0.0 if cb == 0.0 else f32(w / cb)
            best, bestd = 0, None
            for i, lv in enumerate(levels):
                d = abs(x - lv)
                if bestd is None or d < bestd or (d == bestd and lv < levels[best]):
                    best, bestd = i, d
            codes.append(best)
    bits = {16: 4, 8: 3, 4: 2}[len(levels)]
    packed = pack_kbit(codes, bits)
    q8, steps = [], []
    for g in range(0, nb, dq_blocksize):
        grp = c[g:g + dq_blocksize]
        s = max(grp)
        st = f32(s / 255.0)
        steps.append(st)
        for cb in grp:
            if st == 0.0:
                q8.append(0)
            else:
                r = f32(cb / st)
                q = round(r)  # Python round() is half-to-even
                q8.append(min(255, int(q)))
    return packed, q8, steps


def dequantize(packed, q8, steps, levels, blocksize=64, dq_blocksize=256):
    """Returns the bf16 bit patterns of W_hat, flat, row-major."""
    bits = {16: 4, 8: 3, 4: 2}[len(levels)]
    n = len(packed) * 8 // bits
    out = []
    for e, code in enumerate(unpack_kbit(packed, bits, n)):
        b = e // blocksize
        chat = f32(float(q8[b]) * steps[b // dq_blocksize])
        out.append(bf16_bits(f32(levels[code] * chat)))
    return out
