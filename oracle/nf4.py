"""NF4 quantizer oracle (numpy, vectorized).  Test infrastructure only.

What the pages fix, and where:

* NF4 puts its 16 levels at quantiles of the normal distribution so that
  every level stands for an equal share of normally distributed weights
  ("QLoRA: fine-tuning a 65B model on one GPU", section "NormalFloat, double
  quantization, paged optimizers"; "QLoRA: efficient finetuning of quantized
  LLMs", Abstract, item (a)).
* Blockwise quantization keeps one scaling constant per block of weights; the
  constant is the block's absmax ("Qlora 4 Bit Quantization With Nf4 Fp4 Data
  Types And Lora Adapters", entry on 4-bit quantization with the nf4 data
  type).
* Double quantization stores those constants in 8 bits under a second,
  coarser level of constants (blog section "NormalFloat, double quantization,
  paged optimizers"; CoChat Abstract, item (b)).
* The base is quantized once and dequantized to 16 bits on every forward and
  backward pass (blog section "Where the memory goes").

k-bit NormalFloat (NF3, NF2): the ModuLoRA abstract ("ModuLoRA: Finetuning
2-Bit LLMs on Consumer GPUs by Integrating with Modular Quantizers") finetunes
through 2-, 3- and 4-bit weights with a backward pass that materializes the
low-precision weight from whatever quantizer produced it.  Here the 2- and
3-bit types are NormalFloat built the NF4 way with 2^k levels (see
``nfk_levels_f64``), under the same blockwise absmax and double quantization;
the codes are packed densely at k bits per weight (see ``pack_codes_k``).

FP4, the other data type the capability page "Qlora 4 Bit Quantization With
Nf4 Fp4 Data Types And Lora Adapters" names in its title (and the plain
4-bit float NF4 is compared against in the blog section "NormalFloat, double
quantization, paged optimizers"), goes through the same blockwise absmax,
double quantization and storage; only the 16 values behind the codes differ.
The pages give no bit layout for it; it is read as the E2M1 format (see
``fp4_values``).

A caller's codebook ("user4", "user3", "user2"): the ModuLoRA abstract's
backward materializes the weight from a black-box quantizer, so the kernels
must work with whatever 2^k values stand behind the codes.  The oracle
quantizes to such a codebook by its definition, the nearest value with ties
to the lower value (``nearest_code_exact``), under the same block scaling,
double quantization and storage.

Readings taken where the pages are silent (each is listed in the design
notes): level offset delta = 1 - (1/30 + 1/32)/2 with 7 negative levels, an
exact zero and 8 positive levels; blocks of 64 consecutive row-major
elements; nearest level with ties to the lower index; even element in the
low nibble; unsigned linear 8-bit constants per group of 256 consecutive
blocks under an fp32 step max/255, rounded half-to-even; dequantization
w = bf16_rne(fl32(level * fl32(q * step))).
"""

import math
import os

import numpy as np

BLOCKSIZE = 64
DQ_BLOCKSIZE = 256


# --------------------------------------------------------------------------
# Normal quantile function, from its definition
# --------------------------------------------------------------------------

def normal_cdf(x: float) -> float:
    """Phi(x) = P(Z <= x) for a standard normal Z, via the complementary
    error function: Phi(x) = erfc(-x / sqrt 2) / 2."""
    return 0.5 * math.erfc(-x / math.sqrt(2.0))


def normal_quantile(p: float) -> float:
    """Phi^{-1}(p) for 0.5 <= p < 1, by bisection on the monotone Phi.

    Bisection stops when the midpoint of the bracket equals one of its ends,
    i.e. the bracket is two adjacent doubles.  The result is then within one
    ulp of the root of the computed Phi, which is accurate to a few ulp.
    """
    if not (0.5 <= p < 1.0):
        raise ValueError("normal_quantile is only needed on [0.5, 1)")
    lo, hi = 0.0, 40.0
    while True:
        mid = 0.5 * (lo + hi)
        if mid == lo or mid == hi:
            break
        if normal_cdf(mid) < p:
            lo = mid
        else:
            hi = mid
    # pick the end whose Phi is closer to p
    return lo if abs(normal_cdf(lo) - p) <= abs(normal_cdf(hi) - p) else hi


# --------------------------------------------------------------------------
# The 16 NF4 levels
# --------------------------------------------------------------------------

NF4_DELTA = 1.0 - 0.5 * (1.0 / 30.0 + 1.0 / 32.0)


def nf4_levels_f64() -> np.ndarray:
    """The 16 NF4 levels in fp64, sorted ascending.

    Levels sit at normal quantiles (blog section "NormalFloat, double
    quantization, paged optimizers").  Phi^{-1}(1) is infinite, so the
    outermost probability is pulled in to delta.  An exact zero splits the
    levels into 8 positive ones at probabilities evenly spaced from delta
    down to (but not including) 1/2, and 7 negative ones mirrored from 7
    evenly spaced probabilities on the same interval.  Dividing by
    Phi^{-1}(delta) puts the outermost levels at exactly -1 and +1.
    """
    d = NF4_DELTA
    pos = [normal_quantile(d - (d - 0.5) * i / 8.0) for i in range(8)]
    neg = [-normal_quantile(d - (d - 0.5) * j / 7.0) for j in range(7)]
    top = normal_quantile(d)
    vals = sorted(neg + [0.0] + pos)
    return np.array([v / top for v in vals], dtype=np.float64)


def nf4_levels() -> np.ndarray:
    """The NF4 levels rounded once to fp32 (round to nearest even)."""
    return nf4_levels_f64().astype(np.float32)


# --------------------------------------------------------------------------
# k-bit NormalFloat
# --------------------------------------------------------------------------

def nfk_delta(k: int) -> float:
    """Outermost probability of the k-bit type: the average of the centres
    of the last bins of a (2^k - 1)-bin and a 2^k-bin grid on [0, 1], the
    same offset as NF4's (k = 4 gives 1 - (1/30 + 1/32)/2)."""
    n = 2 ** k
    return 1.0 - 0.5 * (1.0 / (2 * (n - 1)) + 1.0 / (2 * n))


def nfk_levels_f64(k: int) -> np.ndarray:
    """The 2^k NormalFloat levels for k = 2, 3, 4 in fp64, ascending.

    Reading (the pages give the construction only for 4 bits): an exact
    zero, 2^(k-1) positive levels at probabilities evenly spaced from delta
    down to (not including) 1/2, and 2^(k-1) - 1 negative levels mirrored
    from evenly spaced probabilities on the same interval, all divided by
    Phi^{-1}(delta) so that the outermost are -1 and +1.  For k = 4 this is
    ``nf4_levels_f64``.
    """
    if k not in (2, 3, 4):
        raise ValueError("k must be 2, 3 or 4")
    d = nfk_delta(k)
    half = 2 ** (k - 1)
    pos = [normal_quantile(d - (d - 0.5) * i / half) for i in range(half)]
    neg = [-normal_quantile(d - (d - 0.5) * j / (half - 1)) for j in range(half - 1)]
    top = normal_quantile(d)
    return np.array([v / top for v in sorted(neg + [0.0] + pos)], dtype=np.float64)


def nfk_levels(k: int) -> np.ndarray:
    """The k-bit NormalFloat levels rounded once to fp32."""
    return nfk_levels_f64(k).astype(np.float32)


# --------------------------------------------------------------------------
# FP4 (E2M1) values
# --------------------------------------------------------------------------

def fp4_values_f64() -> np.ndarray:
    """The value of each 4-bit FP4 code, in code order, in fp64.

    Reading of "fp4" (the pages name the type without a layout): the E2M1
    format.  Bit 3 is the sign, bits 2..1 an exponent e with bias 1, bit 0 a
    mantissa bit m.  e = 0 is subnormal, m / 2; otherwise 2^(e-1) (1 + m/2).
    The magnitudes are then 0, 1/2, 1, 3/2, 2, 3, 4, 6; they are divided by
    6 so that the largest is 1, like the NF4 levels, since a block is scaled
    by its absmax.  Code 8 is -0.
    """
    out = []
    for code in range(16):
        sign = -1.0 if code & 8 else 1.0
        e = (code >> 1) & 3
        m = code & 1
        mag = m / 2.0 if e == 0 else 2.0 ** (e - 1) * (1.0 + m / 2.0)
        out.append(sign * mag / 6.0)
    return np.array(out, dtype=np.float64)


def fp4_values() -> np.ndarray:
    """The FP4 values rounded once to fp32 (round to nearest even)."""
    return fp4_values_f64().astype(np.float32)


CODE_TYPES = ("nf4", "fp4", "nf3", "nf2")
USER_CODES = ("user4", "user3", "user2")
CODE_BITS = {"nf4": 4, "fp4": 4, "nf3": 3, "nf2": 2, "user4": 4, "user3": 3, "user2": 2}
USER_MIN_MAGNITUDE = 2.0 ** -20


def code_bits(code: str) -> int:
    if code not in CODE_BITS:
        raise ValueError(f"unknown code type {code!r}")
    return CODE_BITS[code]


def user_values(code: str, levels) -> np.ndarray:
    """A caller's codebook as fp32, checked against the contract: 2^bits
    finite values with |v| <= 1 and v = 0 or |v| >= 2^-20.  Under it the sum
    of two values is exact in fp64 (their bits span at most 45 places), so
    every midpoint is exact."""
    f = np.asarray(levels, dtype=np.float64).astype(np.float32)  # rounded to fp32
    if f.shape != (2 ** code_bits(code),):
        raise ValueError(f"{code} takes {2 ** code_bits(code)} values")
    if not np.all(np.isfinite(f)):
        raise ValueError("codebook values must be finite")
    a = np.abs(f.astype(np.float64))
    if np.any(a > 1.0) or np.any((a != 0) & (a < USER_MIN_MAGNITUDE)):
        raise ValueError("codebook values need |v| <= 1 and v = 0 or |v| >= 2^-20")
    return f


def code_values(code: str = "nf4", levels=None) -> np.ndarray:
    """fp32 value of each of the 2^bits codes of a code type, in code order
    (for a user code type, the caller's ``levels``)."""
    if code in USER_CODES:
        return user_values(code, levels)
    if code == "nf4":
        return nf4_levels()
    if code == "fp4":
        return fp4_values()
    if code == "nf3":
        return nfk_levels(3)
    if code == "nf2":
        return nfk_levels(2)
    raise ValueError(f"unknown code type {code!r}")


# --------------------------------------------------------------------------
# bf16 helpers
# --------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest, ties to even) and return the
    16-bit patterns.  Written with integer operations on the fp32 bit
    pattern: add 0x7FFF plus the lowest kept bit, then drop 16 bits.  Exact
    for every finite input, subnormals included (NaN is outside the
    contract)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    keep_lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + keep_lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact)."""
    u = np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32)


# --------------------------------------------------------------------------
# Quantizer
# --------------------------------------------------------------------------

def nearest_level(x: np.ndarray, levels_f32: np.ndarray) -> np.ndarray:
    """Index of the level nearest to each fp32 x, ties to the lower index.

    Distances are taken in fp64.  For fp32 operands of nearby magnitude the
    difference is exact in fp64, which is the only case where two distances
    can tie or nearly tie; far from a midpoint, rounding in fp64 cannot
    change which distance is smaller.  ``argmin`` returns the first minimum,
    which is the lower index.  Chunks are independent and are spread over a
    few threads (numpy releases the GIL inside the ufuncs).
    """
    L = levels_f32.astype(np.float64)
    xs = np.asarray(x, dtype=np.float32)
    out = np.empty(xs.shape, dtype=np.uint8)
    flat_in = xs.reshape(-1)
    flat_out = out.reshape(-1)
    chunk = 1 << 19

    def work(s):
        xc = flat_in[s:s + chunk].astype(np.float64)
        d = np.abs(xc[:, None] - L[None, :])
        flat_out[s:s + chunk] = np.argmin(d, axis=1).astype(np.uint8)

    starts = range(0, flat_in.size, chunk)
    if flat_in.size <= 4 * chunk:
        for s in starts:
            work(s)
    else:
        from concurrent.futures import ThreadPoolExecutor
        nthreads = max(1, min(8, len(os.sched_getaffinity(0))))
        with ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(work, starts))
    return out


def nearest_code(x: np.ndarray, values_f32: np.ndarray) -> np.ndarray:
    """Code whose value is nearest to each fp32 x, for values in any code
    order: ties go to the lower value, and of two codes with the same value
    (FP4's +0 and -0) the lower code is taken.  The codes are put in
    ascending order of (value, code) and ``nearest_level`` picks in that
    order; for the ascending NF4 levels this is ``nearest_level`` itself."""
    v = np.asarray(values_f32, dtype=np.float32)
    order = np.lexsort((np.arange(v.size), v.astype(np.float64)))
    return order[nearest_level(x, v[order])].astype(np.uint8)


def nearest_code_exact(x: np.ndarray, values_f32: np.ndarray) -> np.ndarray:
    """Code whose value is nearest to each fp32 x, ties to the lower value,
    of equal values the lowest code, decided without any rounded distance:
    x is nearer to the upper of two consecutive distinct values exactly when
    x > their midpoint, and both x and the midpoint (for values under the
    user-codebook contract) are exact in fp64.  So the nearest value is the
    number of midpoints below x, counted in the ascending list."""
    v = np.asarray(values_f32, dtype=np.float32)
    dist = np.unique(v.astype(np.float64))           # ascending, -0 and +0 once
    codes_of = np.array([int(np.flatnonzero(v.astype(np.float64) == d)[0]) for d in dist],
                        dtype=np.uint8)               # lowest code of each value
    mid = (dist[:-1] + dist[1:]) / 2.0
    assert np.array_equal(mid * 2.0 - dist[:-1], dist[1:]), "midpoints must be exact"
    n = np.searchsorted(mid, np.asarray(x, np.float32).astype(np.float64), side="left")
    return codes_of[n]


def block_absmax(W: np.ndarray, blocksize: int = BLOCKSIZE) -> np.ndarray:
    """c_b = max |w| over each block of ``blocksize`` consecutive elements
    of row-major W (exact in fp32)."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W.shape
    if K % blocksize:
        raise ValueError("K must be a multiple of the block size")
    return np.max(np.abs(W.reshape(-1, blocksize)), axis=1)


def normalize(W: np.ndarray, c: np.ndarray, blocksize: int = BLOCKSIZE) -> np.ndarray:
    """x = fl32(w / c_b), IEEE fp32 division; x = 0 where c_b = 0."""
    Wb = np.ascontiguousarray(W, dtype=np.float32).reshape(-1, blocksize)
    cb = c.astype(np.float32)[:, None]
    x = np.zeros_like(Wb)
    nz = np.broadcast_to(cb != 0, Wb.shape)
    np.divide(Wb, np.broadcast_to(cb, Wb.shape), out=x, where=nz)
    return x


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """Two 4-bit codes per byte, element 2j in the low nibble."""
    c = np.ascontiguousarray(codes, dtype=np.uint8).reshape(-1)
    return (c[0::2] | (c[1::2] << np.uint8(4))).astype(np.uint8)


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    p = np.ascontiguousarray(packed, dtype=np.uint8).reshape(-1)
    out = np.empty(p.size * 2, dtype=np.uint8)
    out[0::2] = p & np.uint8(0x0F)
    out[1::2] = p >> np.uint8(4)
    return out


def _kbit_positions(bits: int):
    """For the 64 elements of a block: (word, bit) of each code bit, bit b of
    the code of element e going to bit pos[b][e] of little-endian uint32
    word word[b][e] of the block's 2 k words (k = bits).

    Layout (chosen so that 8 consecutive codes unpack with a few shifts and
    masks): a block is two halves of 32 elements, each half k words; write
    element e = 32 h + 8 g + 2 i + p (g, i in 0..3, p in 0..1).  Code bits 0
    and 1 go to bits 8 i + 2 g and 8 i + 2 g + 1 of word k h + p (the even
    elements of a half in its first word, the odd ones in the second).  For
    k = 3, code bit 2 goes to bit (8 i + 2 + 2 g + p) mod 32 of word 3 h + 2.
    """
    e = np.arange(64)
    h, g, i, p = e >> 5, (e >> 3) & 3, (e >> 1) & 3, e & 1
    word = [bits * h + p, bits * h + p]
    pos = [8 * i + 2 * g, 8 * i + 2 * g + 1]
    if bits == 3:
        word.append(3 * h + 2)
        pos.append((8 * i + 2 + 2 * g + p) % 32)
    return word, pos


def pack_codes_k(codes: np.ndarray, bits: int) -> np.ndarray:
    """Pack codes of ``bits`` bits (4: ``pack_codes``; 3 or 2: the layout of
    ``_kbit_positions``, 8 * bits bytes per 64-element block)."""
    if bits == 4:
        return pack_codes(codes)
    c = np.ascontiguousarray(codes, dtype=np.uint32).reshape(-1, 64)
    words = np.zeros((c.shape[0], 2 * bits), dtype=np.uint32)
    wsel, pos = _kbit_positions(bits)
    for b in range(bits):
        bit = (c >> np.uint32(b)) & np.uint32(1)
        for e in range(64):
            words[:, wsel[b][e]] |= bit[:, e] << np.uint32(pos[b][e])
    return words.astype("<u4").view(np.uint8).reshape(-1)


def unpack_codes_k(packed: np.ndarray, bits: int) -> np.ndarray:
    if bits == 4:
        return unpack_codes(packed)
    w = np.ascontiguousarray(packed, dtype=np.uint8).view("<u4").reshape(-1, 2 * bits)
    out = np.zeros((w.shape[0], 64), dtype=np.uint8)
    wsel, pos = _kbit_positions(bits)
    for b in range(bits):
        for e in range(64):
            out[:, e] |= (((w[:, wsel[b][e]] >> np.uint32(pos[b][e])) & np.uint32(1))
                          << np.uint32(b)).astype(np.uint8)
    return out.reshape(-1)


def double_quantize(c: np.ndarray, dq_blocksize: int = DQ_BLOCKSIZE):
    """Quantize the absmax constants to 8 bits under a coarser fp32 level.

    Groups are ``dq_blocksize`` consecutive block indices (the last group may
    be shorter).  Per group: s = max c_b; step = fl32(s / 255);
    q_b = min(255, rint(fl32(c_b / step))) with round-half-to-even, and
    q_b = 0 when step = 0.  Returns (q8 uint8 [nblocks], step fp32
    [ngroups]).
    """
    c = np.asarray(c, dtype=np.float32)
    nb = c.size
    ng = (nb + dq_blocksize - 1) // dq_blocksize
    step = np.empty(ng, dtype=np.float32)
    q = np.empty(nb, dtype=np.uint8)
    for g in range(ng):
        cg = c[g * dq_blocksize:(g + 1) * dq_blocksize]
        s = np.max(cg)
        st = np.float32(s) / np.float32(255.0)
        step[g] = st
        if st == 0:
            q[g * dq_blocksize:g * dq_blocksize + cg.size] = 0
            continue
        r = np.rint(cg / st)  # fp32 division, then half-to-even rounding
        q[g * dq_blocksize:g * dq_blocksize + cg.size] = np.minimum(r, 255).astype(np.uint8)
    return q, step


def quantize(W: np.ndarray, blocksize: int = BLOCKSIZE, dq_blocksize: int = DQ_BLOCKSIZE,
             code: str = "nf4", levels=None):
    """Block quantization (NF4 by default, or FP4, NF3, NF2, or a caller's
    codebook ``levels`` for the user code types) + double-quant encoding of
    W [N, K] fp32, one absmax constant per `blocksize` consecutive elements
    (a multiple of 64 dividing K).

    Returns (packed codes uint8 [N*K*bits/8], packed in 64-element units
    whatever the block size; q8 uint8 [N*K/blocksize]; step fp32
    [ceil(N*K/blocksize/dq_blocksize)]).
    """
    if blocksize % 64:
        raise ValueError("the block size must be a multiple of 64")
    c = block_absmax(W, blocksize)
    x = normalize(W, c, blocksize)
    if code in USER_CODES:
        codes = nearest_code_exact(x, code_values(code, levels))
    else:
        codes = nearest_code(x, code_values(code))
    packed = pack_codes_k(codes, code_bits(code))
    q8, step = double_quantize(c, dq_blocksize)
    return packed, q8, step


def dequant_constants(q8: np.ndarray, step: np.ndarray, dq_blocksize: int = DQ_BLOCKSIZE) -> np.ndarray:
    """c_hat_b = fl32(q_b * step_g) for every block b in group g."""
    q8 = np.asarray(q8, dtype=np.uint8)
    g = np.arange(q8.size) // dq_blocksize
    return (q8.astype(np.float32) * np.asarray(step, dtype=np.float32)[g]).astype(np.float32)


def dequantize_f32(packed, q8, step, N, K, blocksize=BLOCKSIZE, dq_blocksize=DQ_BLOCKSIZE,
                   code="nf4", levels=None) -> np.ndarray:
    """fl32(value[code] * c_hat_b) as fp32 [N, K], before the bf16 rounding."""
    levels = code_values(code, levels)
    codes = unpack_codes_k(packed, code_bits(code))
    chat = dequant_constants(q8, step, dq_blocksize)
    vals = levels[codes].reshape(-1, blocksize) * chat[:, None]
    return vals.astype(np.float32).reshape(N, K)


def dequantize(packed, q8, step, N, K, blocksize=BLOCKSIZE, dq_blocksize=DQ_BLOCKSIZE,
               code="nf4", levels=None) -> np.ndarray:
    """The dequantized weight W_hat as bf16 bit patterns [N, K] (uint16)."""
    return f32_to_bf16_bits(dequantize_f32(packed, q8, step, N, K, blocksize, dq_blocksize, code,
                                           levels))


def storage_bytes(N: int, K: int, blocksize=BLOCKSIZE, dq_blocksize=DQ_BLOCKSIZE,
                  code="nf4") -> int:
    """Bytes of the quantized state: packed codes + 8-bit constants + fp32 steps."""
    nb = N * K // blocksize
    return N * K * code_bits(code) // 8 + nb + 4 * ((nb + dq_blocksize - 1) // dq_blocksize)
