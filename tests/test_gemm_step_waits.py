"""Static check of the GEMM main loops' step barriers (CPU only: reads the
gfx950 assembly hipcc writes for csrc/qgemm.hip).

Each pipelined step issues its activation tile loads straight into LDS
(`buffer_load_dwordx4 ... lds`) and then the weight loads into registers,
and ends with `s_waitcnt vmcnt(N)` + `s_barrier`.  Vector memory loads
complete in issue order, so the tile is in LDS for the next step only if at
least N loads were issued after the step's last tile load.  A step that
issues fewer (as the forward did when its constant loads became one per
four steps) races: the next step can read a tile that has not landed.  The
race is rarely visible in results, so the invariant is checked on the code.
"""

import os
import re
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "quantized_base_lora_nf4_amd", "csrc", "qgemm.hip")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.fixture(scope="module")
def asm():
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "qgemm.s")
        subprocess.run([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang",
                        "-target-feature", "-Xclang", "-packed-fp32-ops",
                        "-I" + os.path.join(ROOT, "include"), "--cuda-device-only", "-S", SRC,
                        "-o", out], check=True, capture_output=True)
        return open(out).read()


def kernels(text):
    for m in re.finditer(r"^(_Z\S*k_qgemm_(?:fwd|bwd)\S*):", text, re.M):
        end = text.index(".Lfunc_end", m.end())
        body = [l.strip() for l in text[m.end():end].splitlines()]
        yield m.group(1), [l for l in body if l and not l.startswith((";", "."))]


def step_segments(body):
    """Instructions of each step: from the previous barrier to a barrier,
    for every barrier whose segment contains a direct-to-LDS tile load."""
    start = 0
    for i, ins in enumerate(body):
        if not ins.startswith("s_barrier"):
            continue
        seg = body[start:i]
        start = i + 1
        if any(DMA.match(x) for x in seg):
            yield seg


DMA = re.compile(r"buffer_load_dword\S*\s.*\blds\b")
LOAD = re.compile(r"(global|buffer)_load_")


def tile_covered(seg):
    """Some vmcnt(k) after the step's last tile load with at least k loads
    issued between the two."""
    last_dma = max(i for i, x in enumerate(seg) if DMA.match(x))
    loads = 0
    for x in seg[last_dma + 1:]:
        m = re.search(r"vmcnt\((\d+)\)", x)
        if m and int(m.group(1)) <= loads:
            return True
        if LOAD.match(x):
            loads += 1
    return False


def test_every_step_barrier_covers_its_tile_loads(asm):
    checked = 0
    for name, body in kernels(asm):
        for seg in step_segments(body):
            assert tile_covered(seg), f"{name}: a step barrier may run before the tile landed"
            checked += 1
    # both directions, every code type, both forward constant paths
    assert checked >= 8 * 4


def test_main_loops_keep_weight_loads_in_flight(asm):
    """No vmcnt(0) inside a pipelined step that issues weight loads, other
    than the first (the prologue drains) and the last: a full drain there
    would wait for the weight loads meant for later steps and expose the
    memory latency (what the global form of the tile load did).  Steps of
    the MFMA-only waves load nothing but the tile, so vmcnt(0) is exactly
    their tile wait."""
    checked = 0
    for name, body in kernels(asm):
        segs = list(step_segments(body))
        for seg in segs[1:-1]:
            last_dma = max(i for i, x in enumerate(seg) if DMA.match(x))
            if not any(LOAD.match(x) for x in seg[last_dma + 1:]):
                continue
            checked += 1
            assert not any(re.search(r"vmcnt\(0\)", x) for x in seg), name
    assert checked > 0
