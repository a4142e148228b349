#!/usr/bin/env python3
"""Throughput of the frozen-NF4-base + LoRA linear layer on one MI355X.

Step = one forward + backward pass of the layer for every weight of the
workload (default: the LLaMA-7B q_proj 4096x4096 and up_proj 11008x4096
projections, 4096 tokens, LoRA r=64, alpha=16) with inputs resident in HBM.
The quantized weights are built once before timing (quantization is a
one-time cost of the frozen base); it is timed separately and reported
under "extra", as is the few-token (M = 1, 4, 16) forward path on the
8192x8192 and 28672x8192 weights.

Prints ONE JSON line (rank 0, N = 1).  FLOPs per weight and step:
4 M N K + 6 M r (N + K) (no gradient for the frozen W).

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
"""

import argparse
import ctypes
import hashlib
import re
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
HBM_PEAK_GBPS = 8000.0           # MI355X HBM3E, published


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--events-every", type=int, default=2,
                    help="record the kernel events on every n-th timed step (the event "
                         "records themselves cost a few microseconds of stream time)")
    ap.add_argument("--workload", default="llama7b_q_up_M4096_r64")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (for scaling HBM "
                         "counters) and exit")
    ap.add_argument("--cpu-rows", type=int, default=4096,
                    help="token rows of the workload the CPU oracle runs on")
    ap.add_argument("--lq-only", action="store_true",
                    help="only time the low-rank plus quantized initialization (the "
                         "extra 'lq_init') and print it")
    ap.add_argument("--ilp-only", action="store_true",
                    help="only time the configuration error table and plans (the extra "
                         "'ilp') and print it")
    ap.add_argument("--gemv-only", action="store_true",
                    help="only time the few-token forward and the quantizer (the extras "
                         "'gemv', 'quantize', 'code_types') and print them")
    return ap.parse_args()


# hipEventCreateWithFlags flag (hip_runtime_api.h): the event's record takes
# no system-scope fence.  A plain event writes back and invalidates the
# caches when it is recorded; for events that only take timestamps the HIP
# header names this flag as the way to keep that cost (and its effect on the
# next kernel) out of the measured interval.
HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000


class ClockSampler:
    """The GPU's shader (GFX) clock while work runs: amdsmi (the library
    behind amd-smi and rocm-smi) polled from a thread every few
    milliseconds.  The value it returns is refreshed by the GPU's power
    management firmware only about once a second, so only a run of a few
    seconds gives readings taken under that load.  `mhz(after)` is the
    median of the samples taken `after` seconds or later into the run, None
    when amdsmi is not usable here."""

    def __init__(self, period_s=0.005):
        import threading
        self.period, self.samples, self.handle = period_s, [], None
        self._stop, self._thread = threading.Event(), None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self.amdsmi = amdsmi
            self.handle = amdsmi.amdsmi_get_processor_handles()[0]
            self._read()
        except Exception:
            self.handle = None

    def _read(self):
        a = self.amdsmi
        return a.amdsmi_get_clock_info(self.handle, a.AmdSmiClkType.GFX)["clk"]

    def _loop(self):
        t0 = time.perf_counter()
        while not self._stop.is_set():
            try:
                v = self._read()
                if isinstance(v, (int, float)) and v > 0:
                    self.samples.append((time.perf_counter() - t0, float(v)))
            except Exception:
                pass
            self._stop.wait(self.period)

    def __enter__(self):
        if self.handle is not None:
            import threading
            self._stop.clear()
            self._thread = threading.Thread(target=self._loop, daemon=True)
            self._thread.start()
        return self

    def __exit__(self, *exc):
        if self._thread is not None:
            self._stop.set()
            self._thread.join()
            self._thread = None
        return False

    def mhz(self, after=0.0):
        v = [c for t, c in self.samples if t >= after]
        return float(np.median(v)) if v else None


class HipEvents:
    """hipEvent_t pairs through the HIP runtime's C API (the library's
    measurement calls record them around the dominant kernel).  They only
    take timestamps, so they are created without the system-scope fence."""

    def __init__(self):
        import torch  # noqa: F401  (loads the HIP runtime)
        self.rt = ctypes.CDLL("libamdhip64.so")
        self.rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.rt.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
        self.rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.rt.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.rt.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def create(self):
        e = ctypes.c_void_p()
        assert self.rt.hipEventCreateWithFlags(ctypes.byref(e), HIP_EVENT_DISABLE_SYSTEM_FENCE) == 0
        return e

    def elapsed_ms(self, a, b) -> float:
        assert self.rt.hipEventSynchronize(b) == 0
        ms = ctypes.c_float()
        assert self.rt.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value

    def destroy(self, e):
        self.rt.hipEventDestroy(e)


def kernel_source_hash(names):
    """Hash of the kernel sources' code: comments and blank lines are
    removed first, so that editing a comment keeps the counters valid."""
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "quantized_base_lora_nf4_amd", "csrc", n)) as f:
            h.update(strip_comments(f.read()).encode())
    return h.hexdigest()[:16]


def strip_comments(src: str) -> str:
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    return "\n".join(l.rstrip() for l in src.splitlines() if l.strip())


def load_traffic(kernel: str, workload: str, src_hash: str):
    """HBM bytes per launch from rocprofv3 FETCH_SIZE/WRITE_SIZE runs, stored
    in profiles/traffic.json together with the hash of the kernel sources the
    counters were taken on; null once the sources have changed."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            d = json.load(f)
        e = d[kernel][workload]
        if e.get("src_hash") != src_hash:
            return None
        return e["bytes_per_launch"]
    except (OSError, KeyError, ValueError):
        return None


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this build measures the layer on a single "
              "MI355X (a data-parallel run would add an all-reduce of dA and dB).", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.lq_only or args.ilp_only:
        import quantized_base_lora_nf4_amd as qn
        print(json.dumps({"lq_init": run_lq(qn, torch)} if args.lq_only else
                         {"ilp": run_ilp(qn, torch)}))
        return
    if args.gemv_only:
        import quantized_base_lora_nf4_amd as qn
        qn.lib()
        ev = HipEvents()
        dev = "cuda"

        def d16(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)
        print(json.dumps(run_extras(qn, qn.lib(), ev, torch, dev,
                                    torch.cuda.current_stream().cuda_stream, d16)))
        return
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": 1 << 30, "launches": 4}))
        return
    import quantized_base_lora_nf4_amd as qn
    import workloads as wl_mod

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    qn.lib()
    wl = {w.name: w for w in wl_mod.WORKLOADS}[args.workload]
    assert not wl.fwd_only, "the headline workload is forward + backward"
    dev = "cuda"
    sp = torch.cuda.current_stream().cuda_stream
    L = qn.lib()
    ev = HipEvents()

    def d16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)

    # ---- headline: the fused step on rotated weight copies (cold Infinity
    # Cache), inputs resident in HBM; kernel events recorded live ----
    fx = FusedWorkload(qn, torch, ev, wl, d16, dev, rotate=True)
    head = fx.run(args.steps, args.warmup, args.events_every, sp)
    M, r = wl.M[0], wl.r
    src_hash = kernel_source_hash(["qgemm.hip", "common.hpp"])
    roofline = dict(head["roofline"])
    roofline["traffic"] = load_traffic(roofline["kernel"], wl.name, src_hash)

    extra = {}
    if not args.no_extra:
        # The spec peak is 4096 flop per CU per clock at 2.4 GHz; next to it,
        # the same peak at the shader clock the GPU holds under this step
        mhz = clock_under_load(fx, sp)
        roofline["observed_clock_ghz"] = None if mhz is None else round(mhz / 1e3, 3)
        roofline["peak_at_observed_clock"] = (
            None if mhz is None else round(fx.cus * 4096 * mhz * 1e6 / 1e12, 1))
        roofline["frac_at_observed_clock"] = (
            None if mhz is None else round(roofline["achieved"] / roofline["peak_at_observed_clock"], 4))
        # the same step without rotation (weights may be served from the
        # Infinity Cache), labeled as such
        extra["warm_step"] = fx.run(args.steps, args.warmup, 0, sp, rotate=False)["summary"]
        extra["workloads"] = run_workloads(qn, torch, ev, d16, dev, sp, args)
        extra.update(run_extras(qn, L, ev, torch, dev, sp, d16))
        for code in ("fp4", "nf3", "nf2"):
            extra["code_types"][code]["fused_step"] = code_step(
                qn, L, torch, fx.layers, M, r, wl.s, sp, args.steps, args.warmup,
                head["flops_step"], code)
        import workloads as wl_mod
        book = wl_mod.draw_codebook(wl_mod.rng_for(77, 0), 4, "plain")
        extra["code_types"]["user4"] = {"fused_step": code_step(
            qn, L, torch, fx.layers, M, r, wl.s, sp, args.steps, args.warmup,
            head["flops_step"], "user4", levels=book)}
        extra["block_sizes"] = {
            f"nf4/{bs}": code_step(qn, L, torch, fx.layers, M, r, wl.s, sp, args.steps,
                                   args.warmup, head["flops_step"], "nf4", bs)
            for bs in (128, 256)}
        extra["bf16_gemm_reference"] = run_gemm_reference(torch, fx.layers, M,
                                                          head["per_launch"])
        extra["lq_init"] = run_lq(qn, torch)
        extra["ilp"] = run_ilp(qn, torch)
    host_inputs = fx.host_inputs
    del fx
    torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(host_inputs, wl, args.cpu_rows)

    out = {
        "metric": "fused NF4+LoRA linear fwd+bwd TFLOP/s (% bf16 MFMA peak); GEMV GB/s",
        "value": head["summary"]["TFLOP/s"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["summary"]["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "tokens": M, "r": r, "alpha": wl.alpha,
                   "weights": [f"{w_.name} {w_.N}x{w_.K}" for w_ in wl.weights],
                   "nf4": "blocksize 64, double-quant 256 (8-bit constants, fp32 steps)",
                   "pct_bf16_mfma_peak": head["summary"]["pct_bf16_mfma_peak"],
                   "weight_copies_rotated": head["summary"]["weight_copies_rotated"],
                   "wall_s_timed": head["summary"]["wall_s_timed"]},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(out), flush=True)


ROTATE_BYTES = 512e6   # rotated weight state per workload: twice the 256 MB Infinity Cache
MAX_COPIES = 64


class FusedWorkload:
    """One forward + backward workload: seeded host inputs, device inputs
    and outputs, and `copies` quantized copies of each weight (rotated step
    by step so that no step's weights are served from the Infinity Cache;
    at most MAX_COPIES, so a tiny workload stays warm)."""

    def __init__(self, qn, torch, ev, wl, d16, dev, rotate=True, keep_host=True):
        import workloads as wl_mod
        self.qn, self.torch, self.ev, self.wl = qn, torch, ev, wl
        self.cus = torch.cuda.get_device_properties(0).multi_processor_count
        M, r = wl.M[0], wl.r
        self.layers = []
        self.host_inputs = []
        state = sum(qn.storage_bytes(sp_.N, sp_.K) for sp_ in wl.weights)
        self.copies = int(min(MAX_COPIES, max(1, np.ceil(ROTATE_BYTES / state)))) if rotate else 1
        for wi, spec in enumerate(wl.weights):
            inp = wl_mod.draw_workload_weight(wl, wi)
            if keep_host:
                self.host_inputs.append(inp)
            W = torch.from_numpy(inp.W).to(dev)
            ws = [qn.nf4_quantize(W) for _ in range(self.copies)]
            N, K = spec.N, spec.K
            t = dict(spec=spec, w=ws[0], ws_all=ws, Wf32=W, X=d16(inp.X), dY=d16(inp.dY),
                     A=d16(inp.A), B=d16(inp.B),
                     U=torch.empty(M, r, dtype=torch.int16, device=dev),
                     Y=torch.empty(M, N, dtype=torch.int16, device=dev),
                     dX=torch.empty(M, K, dtype=torch.int16, device=dev),
                     dA=torch.empty(r, K, dtype=torch.int16, device=dev),
                     dB=torch.empty(N, r, dtype=torch.int16, device=dev))
            t["wsf"] = torch.empty(qn.workspace_size(M, N, K, r, False), dtype=torch.uint8,
                                   device=dev)
            t["wsb"] = torch.empty(qn.workspace_size(M, N, K, r, True), dtype=torch.uint8,
                                   device=dev)
            t["st"] = [w.struct() for w in ws]
            self.layers.append(t)
        torch.cuda.synchronize()

    def flops(self):
        M, r = self.wl.M[0], self.wl.r
        step = fwd = bwd = 0.0
        for t in self.layers:
            N, K = t["spec"].N, t["spec"].K
            step += 4.0 * M * N * K + 6.0 * M * r * (N + K)
            fwd += 2.0 * M * N * (K + r)      # X W^T + (sU) B^T
            bwd += 2.0 * M * K * (N + r)      # dY W + dU A
        return step, fwd, bwd

    def run(self, steps, warmup, events_every, sp, rotate=True):
        """Times exactly `steps` steps after `warmup` untimed ones.  With
        events_every > 0 the dominant kernels of every n-th timed step are
        bracketed by events recorded on the launch stream."""
        from quantized_base_lora_nf4_amd._lib import check
        torch, L, ev = self.torch, self.qn.lib(), self.ev
        M, r, s = self.wl.M[0], self.wl.r, self.wl.s
        copies = self.copies if rotate else 1
        nev = steps if events_every else 0
        evs = [[[ev.create() for _ in range(4)] for _ in range(nev)] for _ in self.layers]

        def p(x):
            return x.data_ptr() if x is not None else None

        def step(i, k):
            for li, t in enumerate(self.layers):
                timed = i is not None and events_every and i % events_every == 0
                e = evs[li][i] if timed else [None] * 4
                st = t["st"][k % copies]
                check(L.qlora_linear_fwd_ev(ctypes.byref(st), p(t["X"]), M, p(t["A"]), p(t["B"]),
                                            r, s, p(t["Y"]), p(t["U"]), p(t["wsf"]),
                                            t["wsf"].numel(), sp, e[0], e[1]), "fwd")
                check(L.qlora_linear_bwd_ev(ctypes.byref(st), p(t["X"]), p(t["dY"]), M, p(t["A"]),
                                            p(t["B"]), p(t["U"]), r, s, p(t["dX"]), p(t["dA"]),
                                            p(t["dB"]), p(t["wsb"]), t["wsb"].numel(), sp, e[2],
                                            e[3]), "bwd")

        for k in range(warmup):
            step(None, k)
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        t0.record()
        for i in range(steps):
            step(i, warmup + i)
        t1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        ms_step = t0.elapsed_time(t1) / steps
        flops_step, flops_fwd, flops_bwd = self.flops()
        tflops = flops_step / (ms_step * 1e-3) / 1e12
        summary = {"ms_per_step": round(ms_step, 4), "TFLOP/s": round(tflops, 2),
                   "pct_bf16_mfma_peak": round(100 * tflops / MFMA_BF16_PEAK_TFLOPS, 2),
                   "steps": steps, "weight_copies_rotated": copies,
                   "wall_s_timed": round(wall, 4)}
        out = {"summary": summary, "flops_step": flops_step}
        if not events_every:
            return out
        kt = {"fwd": [0.0, 0], "bwd": [0.0, 0]}
        per_launch = {"fwd": [], "bwd": []}
        for li, t in enumerate(self.layers):
            lf, lb = [], []
            for i, e in enumerate(evs[li]):
                if i % events_every:
                    continue
                f_ms, b_ms = ev.elapsed_ms(e[0], e[1]), ev.elapsed_ms(e[2], e[3])
                kt["fwd"][0] += f_ms
                kt["fwd"][1] += 1
                kt["bwd"][0] += b_ms
                kt["bwd"][1] += 1
                lf.append(f_ms * 1e3)
                lb.append(b_ms * 1e3)
            per_launch["fwd"].append(lf)
            per_launch["bwd"].append(lb)
        for row in evs:
            for e4 in row:
                for e in e4:
                    ev.destroy(e)
        nl = len(self.layers)
        fwd_ms = kt["fwd"][0] / max(1, kt["fwd"][1]) * nl   # per step
        bwd_ms = kt["bwd"][0] / max(1, kt["bwd"][1]) * nl
        fwd_tf = flops_fwd / (fwd_ms * 1e-3) / 1e12
        bwd_tf = flops_bwd / (bwd_ms * 1e-3) / 1e12
        if bwd_ms >= fwd_ms:   # the dominant kernel: the larger share of the step
            dom, dom_tf, dom_us = "k_qgemm_bwd", bwd_tf, bwd_ms / nl * 1e3
        else:
            dom, dom_tf, dom_us = "k_qgemm_fwd", fwd_tf, fwd_ms / nl * 1e3
        out["per_launch"] = per_launch
        out["roofline"] = {
            "bound": "mfma", "kernel": dom, "achieved": round(dom_tf, 1),
            "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(dom_tf / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
            "avg_launch_us": round(dom_us, 1),
            "other": {"k_qgemm_fwd": {"TFLOP/s": round(fwd_tf, 1), "ms_per_step": round(fwd_ms, 4)},
                      "k_qgemm_bwd": {"TFLOP/s": round(bwd_tf, 1), "ms_per_step": round(bwd_ms, 4)},
                      "lora_and_other_ms_per_step": round(ms_step - fwd_ms - bwd_ms, 4),
                      "launch_us_p10_p50_p90": {
                          f"{kn} {t['spec'].name}": [round(float(np.percentile(v, q)), 1)
                                                    for q in (10, 50, 90)]
                          for kn, key in (("k_qgemm_fwd", "fwd"), ("k_qgemm_bwd", "bwd"))
                          for t, v in zip(self.layers, per_launch[key])},
                      "events_on_every_nth_step": events_every},
        }
        return out


def clock_under_load(fx, sp, seconds=3.0, settle=1.5):
    """Median shader clock (MHz) while the step runs back to back for
    `seconds` (untimed, rotated weight copies), from the readings taken
    after the first `settle` seconds; None without amdsmi."""
    clock = ClockSampler()
    if clock.handle is None:
        return None
    t0 = time.perf_counter()
    with clock:
        while time.perf_counter() - t0 < seconds:
            fx.run(100, 0, 0, sp)
    return clock.mhz(after=settle)


# The other forward + backward workloads, reported under extra.workloads:
# (name, timed steps, warmup steps, CPU sample: weight rows, token rows).
EXTRA_WORKLOADS = (("single_1024x1024_M256_r8", 50, 10, 1024, 256),
                   ("llama65b_mlp_M4096_r64", 10, 3, 512, 256),
                   ("llama13b_block_M2048_r64", 20, 5, 1024, 256))


def run_workloads(qn, torch, ev, d16, dev, sp, args):
    """Every other forward + backward workload at full size, on rotated
    weight copies: step time and TFLOP/s, the dominant kernel's roofline,
    and the CPU oracle on a bounded sample (the first weight rows and token
    rows of every weight).  The LLaMA-13B block also times its one-time
    quantization of all seven weights."""
    import workloads as wl_mod
    out = {}
    for name, steps, warmup, wrows, trows in EXTRA_WORKLOADS:
        wl = {w.name: w for w in wl_mod.WORKLOADS}[name]
        fx = FusedWorkload(qn, torch, ev, wl, d16, dev, rotate=True)
        res = fx.run(steps, warmup, 2, sp)
        entry = dict(res["summary"])
        entry["roofline"] = res["roofline"]
        if name == "llama13b_block_M2048_r64":
            entry["quantize_all_weights"] = time_quantize_all(qn, torch, fx)
        host = fx.host_inputs
        del fx, res
        torch.cuda.empty_cache()
        if not args.no_cpu_baseline:
            entry["cpu_baseline"] = cpu_baseline_sample(host, wl, wrows, trows)
        del host
        out[name] = entry
    return out


def time_quantize_all(qn, torch, fx, reps=5):
    """One-time quantization of every weight of the workload (fp32 W
    resident in HBM, 1.3 GB for the LLaMA-13B block, more than the Infinity
    Cache): median of `reps` passes over all weights, after one warm-up."""
    ts = []
    for i in range(reps + 1):
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for t in fx.layers:
            qn.nf4_quantize(t["Wf32"], out=t["ws_all"][i % len(t["ws_all"])])
        e1.record()
        torch.cuda.synchronize()
        if i:
            ts.append(e0.elapsed_time(e1))
    ms = float(np.median(ts))
    nbytes = sum(4 * t["spec"].N * t["spec"].K + qn.storage_bytes(t["spec"].N, t["spec"].K)
                 for t in fx.layers)
    return {"weights": len(fx.layers), "ms": round(ms, 3), "bytes_read_plus_written": nbytes,
            "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "frac_hbm": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}


def run_gemm_reference(torch, layers, M, per_launch, reps=50):
    """Context, not part of the path: a plain bf16 GEMM (torch.matmul, i.e.
    the vendor BLAS) at the four shapes of the step (forward X W^T and
    backward dY W per weight), random bf16 operands already in bf16, no
    dequantization and no adapter, next to the fused kernels' median launch
    times from the timed region."""
    out = []
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    for li, t in enumerate(layers):
        N, K = t["spec"].N, t["spec"].K
        for kind, (rows, cols, depth) in (("fwd", (M, N, K)), ("bwd", (M, K, N))):
            a = torch.randn(rows, depth, device="cuda", dtype=torch.bfloat16, generator=g)
            b = torch.randn(cols, depth, device="cuda", dtype=torch.bfloat16, generator=g)
            for _ in range(5):
                c = a @ b.t()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                c = a @ b.t()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) / reps * 1e3
            ours = float(np.median(per_launch[kind][li]))
            out.append({"shape_MxNxK": f"{rows}x{cols}x{depth}", "for": f"{kind} {t['spec'].name}",
                        "bf16_blas_us": round(us, 1),
                        "bf16_blas_TFLOP/s": round(2 * rows * cols * depth / us / 1e6, 1),
                        "fused_nf4_lora_us": round(ours, 1)})
            del a, b, c
    torch.cuda.empty_cache()
    return out


LQ_R, LQ_L, LQ_ITERS, LQ_POWER = 64, 80, 2, 2


def run_lq(qn, torch, reps=5):
    """Low-rank plus quantized initialization of the LLaMA-7B q_proj and
    up_proj weights (planted-rank synthetic weights, rank 64, subspace 80,
    2 iterations of 2 power rounds each, NF4): whole-call time, median of
    `reps` calls after one warm-up."""
    import workloads as wl_mod
    out = []
    for wi, (N, K) in enumerate(((4096, 4096), (11008, 4096))):
        inp = wl_mod.draw_lq_inputs(N, K, LQ_R, LQ_L, seed=0, index=wi)
        W = torch.from_numpy(inp.W).cuda()
        Om = torch.from_numpy(inp.Omega).cuda()
        ws = torch.empty(qn.lq_workspace_size(N, K, LQ_R, LQ_L), dtype=torch.uint8, device="cuda")
        ts = []
        for i in range(reps + 1):
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            qn.lq_init(W, Om, LQ_R, iters=LQ_ITERS, power_iters=LQ_POWER, start="svd", s=0.25,
                       ws=ws)
            e1.record()
            torch.cuda.synchronize()
            if i:
                ts.append(e0.elapsed_time(e1))
        ms = float(np.median(ts))
        # E is streamed by 2 P + 2 products per L step (P power rounds), plus
        # the residual (W in, R out) and the quantizer per Q step, plus the
        # error pass (W and Q in, E out) from the second iteration on
        e_reads = LQ_ITERS * (2 * LQ_POWER + 2)
        flops = LQ_ITERS * (2 * LQ_POWER + 2) * 2.0 * N * K * LQ_L
        out.append({"weight": f"{N}x{K}", "r": LQ_R, "l": LQ_L, "iters": LQ_ITERS,
                    "power_iters": LQ_POWER, "ms": round(ms, 3),
                    "products_TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 2),
                    "E_passes": e_reads})
        del W, Om, ws
        torch.cuda.empty_cache()
    return out


def run_ilp(qn, torch, reps=3):
    """Error table of the LLaMA-13B block (7 matrices, 317M weights) for
    every configuration (four code types x block sizes 64, 128, 256), then
    plans at four average bit budgets.  Per table call: the quantizer reads
    W and writes the state, the error pass reads W and the state again."""
    import workloads as wl_mod
    configs = tuple((c, b) for c in ("nf4", "fp4", "nf3", "nf2") for b in (64, 128, 256))
    wl = wl_mod.LLAMA13B_BLOCK
    Ws = [torch.from_numpy(wl_mod.draw_weight(sp, wl_mod.rng_for(wl.seed, 2000 + i))).cuda()
          for i, sp in enumerate(wl.weights)]
    need = max(int(qn.lib().qlora_config_error_workspace_size(W.shape[0], W.shape[1], 0, 64, 0))
               for W in Ws)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    out = torch.empty(len(Ws) * len(configs), dtype=torch.float64, device="cuda")

    def table():
        for m, W in enumerate(Ws):
            for c, (code, bs) in enumerate(configs):
                qn.quant_error(W, code, ws=ws, out=out[m * len(configs) + c:][:1], blocksize=bs)
    table()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        table()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    ms = float(np.median(ts))
    err = out.cpu().numpy().reshape(len(Ws), len(configs))
    nbytes = np.array([[qn.storage_bytes(W.shape[0], W.shape[1], c, b) for c, b in configs]
                       for W in Ws])
    nw = sum(W.numel() for W in Ws)
    moved = sum(2 * 4 * W.numel() + 2 * int(nbytes[m][c]) for m, W in enumerate(Ws)
                for c in range(len(configs)))
    plans = []
    for bits in (2.3, 2.7, 3.2, 3.7):
        t0 = time.perf_counter()
        got = qn.ilp_plan(err, nbytes, int(nw * bits / 8))
        dt = time.perf_counter() - t0
        plans.append({"bits_per_weight": bits,
                      "choice": [f"{configs[c][0]}/{configs[c][1]}" for c in got[0]],
                      "error_vs_all_nf4_64": round(got[1] / float(err[:, 0].sum()), 4),
                      "plan_ms": round(dt * 1e3, 3)})
    del Ws, ws
    torch.cuda.empty_cache()
    return {"matrices": len(wl.weights), "configs": [f"{c}/{b}" for c, b in configs],
            "weights": nw, "table_ms": round(ms, 3),
            "table_GB/s": round(moved / (ms * 1e-3) / 1e9, 1), "plans": plans}


def code_step(qn, L, torch, layers, M, r, s, sp, steps, warmup, flops_step, code, blocksize=64,
              levels=None):
    """The same fused forward + backward step with the weights quantized to
    another code type, a caller's codebook or another block size (same
    kernels, other code table, code width or constant indexing)."""
    from quantized_base_lora_nf4_amd._lib import check
    qw = [qn.nf4_quantize(t["Wf32"], code=code, blocksize=blocksize, levels=levels)
          for t in layers]
    sts = [w.struct() for w in qw]

    def p(x):
        return x.data_ptr() if x is not None else None

    def one():
        for t, st in zip(layers, sts):
            check(L.qlora_linear_fwd(ctypes.byref(st), p(t["X"]), M, p(t["A"]), p(t["B"]), r, s,
                                     p(t["Y"]), p(t["U"]), p(t["wsf"]), t["wsf"].numel(), sp),
                  f"{code} fwd")
            check(L.qlora_linear_bwd(ctypes.byref(st), p(t["X"]), p(t["dY"]), M, p(t["A"]),
                                     p(t["B"]), p(t["U"]), r, s, p(t["dX"]), p(t["dA"]),
                                     p(t["dB"]), p(t["wsb"]), t["wsb"].numel(), sp), f"{code} bwd")
    for _ in range(warmup):
        one()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        one()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    del qw
    return {"ms_per_step": round(ms, 4), "TFLOP/s": round(flops_step / (ms * 1e-3) / 1e12, 2),
            "steps": steps}


def run_extras(qn, L, ev, torch, dev, sp, d16):
    """Few-token forward (GB/s on the packed weight stream) and one-time
    quantization (GB/s), on rotated weight copies so that no call is served
    from the 256 MB Infinity Cache."""
    from quantized_base_lora_nf4_amd._lib import check
    import workloads as wl_mod
    res = {"gemv": [], "quantize": [], "copy": None,
           "code_types": {c: {"gemv_M1": []} for c in ("fp4", "nf3", "nf2")}}
    # measured streaming reference next to the 8 TB/s spec: a plain 1 GiB
    # device copy (reads 1 GiB, writes 1 GiB; larger than the Infinity Cache)
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    c0 = torch.cuda.Event(enable_timing=True)
    c1 = torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(5):
        dst.copy_(src)
    c1.record()
    torch.cuda.synchronize()
    cms = c0.elapsed_time(c1) / 5
    res["copy"] = {"bytes_read_plus_written": 2 << 30, "us": round(cms * 1e3, 1),
                   "GB/s": round((2 << 30) / (cms * 1e-3) / 1e9, 1)}
    del src, dst
    torch.cuda.empty_cache()
    g = wl_mod.SKINNY_GEMV
    res["hbm_read_ceiling"] = hbm_read_ceiling(
        qn, torch, ev, sp, [qn.storage_bytes(sp_.N, sp_.K) for sp_ in g.weights])
    e0, e1, a0, a1 = ev.create(), ev.create(), ev.create(), ev.create()
    for wi, spec in enumerate(g.weights):
        N, K = spec.N, spec.K
        inp = wl_mod.draw_workload_weight(g, wi, M=max(g.M))
        W = torch.from_numpy(inp.W).to(dev)
        wbytes = N * K // 2 + N * K // 64 + 4 * ((N * K // 64 + 255) // 256)
        ncopy = max(3, int(np.ceil(768e6 / wbytes)))
        copies = [qn.nf4_quantize(W) for _ in range(ncopy)]
        structs = [c.struct() for c in copies]
        # quantize GB/s (fp32 in, codes + constants out)
        qt = []
        for i in range(2 * ncopy):
            ctypes_args = copies[i % ncopy]
            torch.cuda.synchronize()
            s0 = torch.cuda.Event(enable_timing=True)
            s1 = torch.cuda.Event(enable_timing=True)
            s0.record()
            qn.nf4_quantize(W, out=ctypes_args)
            s1.record()
            torch.cuda.synchronize()
            if i >= 2:
                qt.append(s0.elapsed_time(s1))
        qms = float(np.median(qt))
        res["quantize"].append({"weight": f"{N}x{K}", "us": round(qms * 1e3, 1),
                                "GB/s": round((4 * N * K + wbytes) / (qms * 1e-3) / 1e9, 1)})
        A, B = d16(inp.A), d16(inp.B)
        for M in g.M:
            res["gemv"].append(_time_gemv(L, torch, ev, structs, inp, M, N, K, g, A, B, d16, dev,
                                          sp, wbytes, e0, e1))
        # the other code types on the same kernel, one token; GB/s counts
        # each type's own weight bytes
        for code in ("fp4", "nf3", "nf2"):
            del copies, structs
            torch.cuda.empty_cache()
            cb = qn.storage_bytes(N, K, code)
            nc = max(3, int(np.ceil(768e6 / cb)))
            copies = [qn.nf4_quantize(W, code=code) for _ in range(nc)]
            structs = [c.struct() for c in copies]
            res["code_types"][code]["gemv_M1"].append(
                _time_gemv(L, torch, ev, structs, inp, 1, N, K, g, A, B, d16, dev, sp, cb, e0, e1))
        del copies, W
        torch.cuda.empty_cache()
    return res


def _time_gemv(L, torch, ev, structs, inp, M, N, K, g, A, B, d16, dev, sp, wbytes, e0, e1):
    """Few-token forward on rotated weight copies: the weight-streaming
    kernel alone and the whole call.  Calls are issued back to back; each
    call's weight-streaming kernel is bracketed by its own pair of events
    (recorded on the launch stream), so a pair measures the kernel without
    the idle-to-busy dispatch a synchronized single call would add."""
    from quantized_base_lora_nf4_amd._lib import check
    ncopy = len(structs)
    X = d16(inp.X[:M])
    Y = torch.empty(M, N, dtype=torch.int16, device=dev)
    ws = torch.empty(qn_ws(L, M, N, K, g.r), dtype=torch.uint8, device=dev)
    it, warm = 60, 6
    pairs = [(ev.create(), ev.create()) for _ in range(it)]
    for i in range(it + warm):
        st = structs[i % ncopy]
        a, b = pairs[i - warm] if i >= warm else (None, None)
        check(L.qlora_linear_fwd_ev(ctypes.byref(st), X.data_ptr(), M, A.data_ptr(),
                                    B.data_ptr(), g.r, g.s, Y.data_ptr(), None,
                                    ws.data_ptr(), ws.numel(), sp, a, b), "gemv")
        if i == warm - 1:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    kern = [ev.elapsed_ms(a, b) for a, b in pairs]
    for a, b in pairs:
        ev.destroy(a)
        ev.destroy(b)
    # whole call (all launches) on the stream
    for i in range(it + warm):
        st = structs[i % ncopy]
        L.qlora_linear_fwd_ev(ctypes.byref(st), X.data_ptr(), M, A.data_ptr(), B.data_ptr(),
                              g.r, g.s, Y.data_ptr(), None, ws.data_ptr(), ws.numel(), sp,
                              None, None)
        if i == warm - 1:
            torch.cuda.synchronize()
            c0 = torch.cuda.Event(enable_timing=True)
            c0.record()
    c1 = torch.cuda.Event(enable_timing=True)
    c1.record()
    torch.cuda.synchronize()
    call_ms = c0.elapsed_time(c1) / it
    k_ms = float(np.median(kern))
    k_avg = float(np.mean(kern))
    gbs = wbytes / (k_avg * 1e-3) / 1e9
    return {
        "weight": f"{N}x{K}", "M": M, "r": g.r,
        "kernel_us": round(k_ms * 1e3, 2),
        "kernel_us_p10_p90": [round(float(np.percentile(kern, q)) * 1e3, 2) for q in (10, 90)],
        "kernel_GB/s": round(wbytes / (k_ms * 1e-3) / 1e9, 1),
        "kernel_frac_hbm": round(wbytes / (k_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "call_us": round(call_ms * 1e3, 2),
        "call_GB/s": round(wbytes / (call_ms * 1e-3) / 1e9, 1),
        "weight_bytes": wbytes, "copies_rotated": ncopy,
        "roofline": {"bound": "hbm", "kernel": "k_qgemv", "achieved": round(gbs, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBPS, 4), "avg_launch_us": round(k_avg * 1e3, 2),
                     "traffic": load_traffic("k_qgemv", f"skinny_gemv_{N}x{K}_M{M}",
                                             kernel_source_hash(["gemv.hip", "common.hpp"]))}}


def hbm_read_ceiling(qn, torch, ev, sp, sizes, reps=40):
    """The measured HBM read ceiling next to the 8 TB/s spec: a read-only
    stream (qlora_stream_read) over buffers of the few-token weight
    streams' sizes, rotated over copies that together exceed the Infinity
    Cache three times; launches back to back, each between its own events."""
    from quantized_base_lora_nf4_amd._lib import QLORA_STREAM_GRID, check
    L = qn.lib()
    out = []
    sink = torch.empty(QLORA_STREAM_GRID, dtype=torch.int32, device="cuda")
    for nbytes in sizes:
        nb = (int(nbytes) + 15) // 16 * 16
        ncopy = max(3, int(np.ceil(768e6 / nb)))
        bufs = [torch.full((nb,), 1, dtype=torch.uint8, device="cuda") for _ in range(ncopy)]
        pairs = [(ev.create(), ev.create()) for _ in range(reps)]
        for i in range(reps + 4):
            a, b = pairs[i - 4] if i >= 4 else (None, None)
            if a is not None:
                assert ev.rt.hipEventRecord(a, ctypes.c_void_p(sp)) == 0
            check(L.qlora_stream_read(bufs[i % ncopy].data_ptr(), nb, sink.data_ptr(), sp),
                  "stream_read")
            if b is not None:
                assert ev.rt.hipEventRecord(b, ctypes.c_void_p(sp)) == 0
        torch.cuda.synchronize()
        ts = [ev.elapsed_ms(a, b) for a, b in pairs]
        for a, b in pairs:
            ev.destroy(a)
            ev.destroy(b)
        ms = float(np.median(ts))
        out.append({"bytes": nb, "us": round(ms * 1e3, 2),
                    "us_p10_p90": [round(float(np.percentile(ts, q)) * 1e3, 2) for q in (10, 90)],
                    "GB/s": round(nb / (ms * 1e-3) / 1e9, 1),
                    "frac_hbm": round(nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                    "copies_rotated": ncopy})
        del bufs
        torch.cuda.empty_cache()
    return out


def qn_ws(L, M, N, K, r):
    return int(L.qlora_workspace_size(M, N, K, r, 0))


CPU_BASELINE_MIN_S = 10.0
CPU_BASELINE_MAX_PASSES = 20


CPU_SAMPLE_MIN_S = 3.0


def cpu_baseline_sample(host_inputs, wl, wrows, trows):
    """The CPU oracle, as it stands, on a bounded sample of a workload: for
    every weight its first `wrows` rows (quantized by the oracle, untimed)
    and the first `trows` token rows; timed: dequantize + fp64 forward +
    backward (the backward's dA and dX over the sampled weight rows)."""
    from oracle import linear, nf4
    states = []
    for inp in host_inputs:
        Wr = np.ascontiguousarray(inp.W[:wrows])
        states.append((nf4.quantize(Wr), Wr.shape))
    cores = len(os.sched_getaffinity(0))
    flops, passes = 0.0, 0
    t0 = time.perf_counter()
    while True:
        for inp, (st, (N, K)) in zip(host_inputs, states):
            Wh = nf4.bf16_bits_to_f32(nf4.dequantize(*st, N, K))
            X = nf4.bf16_bits_to_f32(inp.X[:trows])
            dY = nf4.bf16_bits_to_f32(inp.dY[:trows, :N])
            A = nf4.bf16_bits_to_f32(inp.A)
            B = nf4.bf16_bits_to_f32(inp.B[:N])
            linear.forward(X, Wh, A, B, wl.s)
            linear.backward(X, dY, Wh, A, B, wl.s)
            flops += 4.0 * trows * N * K + 6.0 * trows * wl.r * (N + K)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= CPU_SAMPLE_MIN_S or passes >= CPU_BASELINE_MAX_PASSES:
            break
    return {"value": round(flops / dt / 1e12, 5), "unit": "TFLOP/s", "cores": blas_threads(cores),
            "kind": "oracle",
            "sample": (f"{wl.name}: first {wrows} rows of each of the {len(host_inputs)} weights, "
                       f"first {trows} of {wl.M[0]} token rows; oracle dequantize + fp64 forward "
                       f"+ backward, {passes} passes ({dt:.1f} s)"),
            "seconds": round(dt, 2)}


def blas_threads(cores):
    try:
        from threadpoolctl import threadpool_info
        info = [d for d in threadpool_info() if d.get("user_api") == "blas"]
        return max([d.get("num_threads", 0) for d in info] + [1])
    except Exception:  # pragma: no cover
        return cores


def cpu_baseline(host_inputs, wl, rows):
    """The CPU oracle, as it stands, on a bounded sample of the same workload:
    dequantize every weight from its (oracle-made) NF4 state, then fp64
    forward + backward of the first `rows` token rows.  Reported in the
    headline unit (TFLOP/s over that sample)."""
    from oracle import linear, nf4
    import workloads as wl_mod
    states = []
    for inp, spec in zip(host_inputs, wl.weights):
        states.append((nf4.quantize(inp.W), spec))
    cores = len(os.sched_getaffinity(0))
    flops = 0.0
    passes = 0
    t0 = time.perf_counter()
    # whole passes over the sample until at least MIN_S seconds of CPU work
    while True:
        for inp, (st, spec) in zip(host_inputs, states):
            N, K = spec.N, spec.K
            Wh = nf4.bf16_bits_to_f32(nf4.dequantize(*st, N, K))
            X = nf4.bf16_bits_to_f32(inp.X[:rows])
            dY = nf4.bf16_bits_to_f32(inp.dY[:rows])
            A = nf4.bf16_bits_to_f32(inp.A)
            B = nf4.bf16_bits_to_f32(inp.B)
            linear.forward(X, Wh, A, B, wl.s)
            linear.backward(X, dY, Wh, A, B, wl.s)
            flops += 4.0 * rows * N * K + 6.0 * rows * wl.r * (N + K)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= CPU_BASELINE_MIN_S or passes >= CPU_BASELINE_MAX_PASSES:
            break
    try:
        from threadpoolctl import threadpool_info
        info = [d for d in threadpool_info() if d.get("user_api") == "blas"]
        blas = ",".join(f"{d.get('internal_api')}" for d in info) or "?"
        threads = max([d.get("num_threads", 0) for d in info] + [1])
    except Exception:  # pragma: no cover
        blas, threads = "?", cores
    return {"value": round(flops / dt / 1e12, 5), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": (f"{wl.name}: all {len(wl.weights)} weights, first {rows} of {wl.M[0]} "
                       f"token rows; oracle dequantize + fp64 forward + backward, "
                       f"{passes} passes ({dt:.1f} s, numpy BLAS {blas}, {threads} threads "
                       f"of {cores} host cores)"),
            "seconds": round(dt, 2)}


if __name__ == "__main__":
    main()
