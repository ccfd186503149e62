#!/usr/bin/env python3
"""Benchmark of the tiled product Out = A . B^T on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--repeats R] [--cpu-seconds S]

A step is one call of the product on the headline workload: bfloat16
8192 x 8192 x 8192, fp32 accumulation, bf16 output (persistent 256 x 256 x 64
tiles), inputs N(0,1)*0.05 from seed 3, already resident in HBM.  The other
measured workloads (MXFP8, MXFP6, MXFP4 and NVFP4 8192^3, bf16 4096^3, 1024
batched 128x256x64 and the 128x64x64 single tile, bf16 8192^3 with both
operands row-major and MXFP8 8192^3 with M/N-major operands) are timed after
it and reported in the same line.

Every workload's inputs are drawn and copied to the device before the first
timed call, so no host work idles the GPU between workloads.  The headline
workload then runs W untimed calls and R repeats of exactly K timed calls
(HIP events on the launch stream, synchronised on both sides); the reported
time is the median repeat.  Each other workload runs max(W, 4K) untimed calls
first (the count is in its entry), so that it is timed at its settled rate
rather than in the transient after the previous workload's clock window.  After its timed repeats (outside them), each workload runs
untimed for 1.5 s while the shader clock and socket power are sampled
(amdsmi; the firmware's table refreshes about once a second): the sustained
clock each number was taken at.  The batched workload (184.5 MB per call,
under the 256 MB last-level cache) rotates over three separate input/output
sets, so every call reads and writes HBM; the others each move 100-400 MB per
call.  A 1 GiB device copy gives the practical HBM ceiling.

Prints ONE JSON line.  `roofline` describes the dominant kernel: achieved =
algorithmic flops per launch / median launch time, against the dense bf16
MFMA peak.  `roofline.traffic` is the HBM bytes per launch measured with
rocprofv3 counters (FETCH_SIZE + WRITE_SIZE, scaled by a copy kernel's
reading) when profiles/traffic.json was taken on the current kernel sources,
else null.  `cpu_baseline` is the fp64 oracle timed on the host on a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GEMM TFLOP/s and % of MFMA dense peak (bf16 8192³; MXFP8 8192³)"
PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "e4m3": 5033.2, "e2m1": 10066.3,
               "e2m3": 10066.3, "e3m2": 10066.3,   # dense MFMA, MI355X (fp6 as fp4)
               "nvfp4": 2516.6}  # NVFP4 runs on the fp16 matrix cores (dequantized in the copies)
HBM_GBS = 8000.0
ORDER = ["bf16_8192", "mxfp8_8192", "mxfp6_8192", "mxfp4_8192", "nvfp4_8192", "bf16_8192_nn",
         "mxfp8_8192_mn", "bf16_4096", "batched", "tile_f16"]
# input/output sets a workload rotates over (more than the 256 MB last-level
# cache holds, so each call streams from HBM)
SETS = {"batched": 3}
def kernel_hash() -> str:
    """Hash of every kernel and host source file of the library (csrc/)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "tensor_core_matrix_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".h", ".hip", ".cpp")):
            with open(os.path.join(csrc, f), "rb") as fh:
                h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # The shader clock ramps up over the first tens of milliseconds of load;
    # 50 untimed calls (about 40 ms of the headline workload) reach the
    # steady state before the timed ones.
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--repeats", type=int, default=5, help="timed repeats of --steps calls; median")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target wall time of the oracle's CPU sample")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the clock/power window after each workload")
    ap.add_argument("--only", default=None,
                    help="time a single workload, or 'copy' (profiling runs)")
    return ap.parse_args(argv)


# ----------------------------------------------------------------------------
# Clock and power during the timed region
# ----------------------------------------------------------------------------
class ClockSampler:
    """Samples the shader clock and socket power of the GPU that torch calls
    device 0 (matched by PCI address through amdsmi) every few milliseconds
    while active.  Gives None where amdsmi or the metrics are unavailable."""

    def __init__(self, torch):
        self.h = None
        self.amdsmi = None
        try:
            import amdsmi

            amdsmi.amdsmi_init()
            props = torch.cuda.get_device_properties(0)
            want = (props.pci_domain_id, props.pci_bus_id, props.pci_device_id)
            handles = amdsmi.amdsmi_get_processor_handles()
            for h in handles:
                bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)  # "dddd:bb:dd.f"
                dom, bus, rest = bdf.split(":")
                dev = rest.split(".")[0]
                if (int(dom, 16), int(bus, 16), int(dev, 16)) == want:
                    self.h = h
            if self.h is None and len(handles) == 1:
                self.h = handles[0]
            self.amdsmi = amdsmi
            self.read()
        except Exception as e:  # no metrics: report null
            print(f"[bench] no clock/power readings ({type(e).__name__}: {e})", file=sys.stderr)
            self.h = None
        self.samples = []
        self._stop = threading.Event()
        self._th = None

    def read(self):
        m = self.amdsmi.amdsmi_get_gpu_metrics_info(self.h)
        clks = m.get("current_gfxclks")
        if isinstance(clks, list):
            clks = [c for c in clks if isinstance(c, (int, float)) and 0 < c < 10000]
        clk = statistics.mean(clks) if clks else m.get("current_gfxclk")
        pw = m.get("current_socket_power")
        if not isinstance(pw, (int, float)):
            pw = m.get("average_socket_power")
        return (float(clk) if isinstance(clk, (int, float)) else None,
                float(pw) if isinstance(pw, (int, float)) else None)

    def _loop(self):
        while not self._stop.is_set():
            try:
                self.samples.append((time.perf_counter(),) + self.read())
            except Exception:
                pass
            time.sleep(0.005)

    def start(self):
        self.samples = []
        if self.h is None:
            return
        self._stop.clear()
        self._th = threading.Thread(target=self._loop, daemon=True)
        self._th.start()

    def stop(self, tail_s=None):
        """Stop sampling; mean clock and power over the samples (the last
        tail_s seconds of them only, when given)."""
        if self._th is None:
            return None
        self._stop.set()
        self._th.join()
        self._th = None
        smp = self.samples
        if tail_s is not None and smp:
            t_end = smp[-1][0]
            smp = [x for x in smp if x[0] >= t_end - tail_s]
        clk = [c for _, c, _ in smp if c]
        pw = [p for _, _, p in smp if p]
        if not clk and not pw:
            return None
        return {"sclk_mhz": round(statistics.mean(clk), 1) if clk else None,
                "sclk_mhz_min": min(clk) if clk else None,
                "sclk_mhz_max": max(clk) if clk else None,
                "power_w": round(statistics.mean(pw), 1) if pw else None,
                "samples": len(smp)}

    def window(self, fn, torch, seconds=1.5, tail_s=0.6, batch=20):
        """Clock and power under sustained calls of fn: untimed calls for
        `seconds`, sampled throughout; the firmware's metrics table refreshes
        only about once a second, so the last tail_s seconds are reported."""
        if self.h is None:
            return None
        self.start()
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            for _ in range(batch):
                fn()
            torch.cuda.synchronize()
        return self.stop(tail_s)


# ----------------------------------------------------------------------------
# Workloads in the launch configuration that is timed (the GPU parity tests
# run the very same calls)
# ----------------------------------------------------------------------------
class Prepared:
    """A workload with its inputs resident on the device.  `fn()` makes one
    call, on input/output set (calls so far) mod `sets`; `outs[s]` is set s's
    output and `host` the CPU inputs (all sets hold the same values)."""

    def __init__(self, w, calls, outs, host, nbytes):
        self.w, self.calls, self.outs, self.host, self.nbytes = w, calls, outs, host, nbytes
        self.sets = len(calls)
        self.i = 0

    def fn(self):
        self.calls[self.i % self.sets]()
        self.i += 1


def _call(w, torch, tcm, x, out):
    """One product of workload w on device inputs x into out, through the entry
    that serves it."""
    if w.dtype == "e4m3" and (w.a_order == "col" or w.b_order == "row"):
        # MXFP8 in another arrangement: the general MX entry on strided views
        av = x["A"] if w.a_order == "row" else x["A"].t()
        bv = x["B"] if w.b_order == "row" else x["B"].t()
        return lambda: tcm.gemm_mx(av, bv, x["SA"], x["SB"], out)
    if w.dtype in ("e4m3", "e2m1"):
        mx = tcm.gemm_mx_fp8 if w.dtype == "e4m3" else tcm.gemm_mx_fp4
        return lambda: mx(x["A"], x["B"], x["SA"], x["SB"], out)
    if w.dtype == "nvfp4":
        ga, gb = w.globals
        return lambda: tcm.gemm_nvfp4(x["A"], x["B"], x["SA"], x["SB"], ga, gb, out)
    if w.dtype in ("e2m3", "e3m2"):
        return lambda: tcm.gemm_mx_fp6(x["A"], x["B"], x["SA"], x["SB"], out, elem=w.dtype)
    if w.batch > 1:
        return lambda: tcm.batched_gemm_tn(x["A"], x["B"], out)
    if w.b_order == "row":
        # A . B with B stored K x N: the general entry, N-major B
        return lambda: tcm.gemm(x["A"], x["B"], out=out)
    return lambda: tcm.gemm_tn(x["A"], x["B"], out)


def prepare(name, torch, inp, tcm, sets=None) -> Prepared:
    w = inp.WORKLOADS[name]
    host = inp.make(w)
    odt = torch.bfloat16 if w.out_dtype == "bf16" else torch.float32
    shape = (w.batch, w.M, w.N) if w.batch > 1 else (w.M, w.N)
    calls, outs = [], []
    for _ in range(sets or SETS.get(name, 1)):
        x = {k: v.to("cuda") for k, v in host.items()}
        out = torch.empty(shape, dtype=odt, device="cuda")
        calls.append(_call(w, torch, tcm, x, out))
        outs.append(out)
    nbytes = sum(v.numel() * v.element_size() for v in host.values()) + \
        outs[0].numel() * outs[0].element_size()
    return Prepared(w, calls, outs, host, nbytes)


def timed(fn, steps, warmup, repeats, torch):
    """ms per call of each of `repeats` runs of `steps` back-to-back calls on
    the current stream, after `warmup` untimed calls."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    reps = []
    for _ in range(repeats):
        torch.cuda.synchronize()
        start.record()
        for _ in range(steps):
            fn()
        stop.record()
        torch.cuda.synchronize()
        reps.append(start.elapsed_time(stop) / steps)
    return reps


def copy_ceiling(torch, steps=20, warmup=5):
    """GB/s of a plain 1 GiB device-to-device copy (read + write counted)."""
    src = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    reps = timed(lambda: dst.copy_(src), steps, warmup, 3, torch)
    ms = statistics.median(reps)
    gbs = 2 * src.numel() * 4 / (ms * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return ms, gbs


def cpu_baseline(target_s: float):
    """The fp64 oracle as it stands, on whole rows of the 8192^3 bf16 product."""
    from oracle import oracle as orc
    from tensor_core_matrix_amd import inputs as inp

    w = inp.WORKLOADS["bf16_8192"]
    x = inp.make(w)
    a, b = inp.raw(x["A"]), inp.raw(x["B"])
    threads = orc.default_threads()

    def run(rows):
        t0 = time.perf_counter()
        orc.gemm_tn(orc.BF16, a[:rows], b, nthreads=threads)
        return time.perf_counter() - t0

    # Each call decodes all of B once, then computes `rows` whole output rows:
    # two short calls give the fixed and the per-row cost, which sizes the
    # measured call to last about target_s.
    r1, r2 = threads, 3 * threads
    t1, t2 = run(r1), run(r2)
    per_row = max((t2 - t1) / (r2 - r1), 1e-6)
    fixed = max(t1 - r1 * per_row, 0.0)
    rows2 = int(max(r2, min(w.M, (target_s - fixed) / per_row)))
    rows2 = max(threads, rows2 - rows2 % threads)
    dt = run(rows2)
    flops = 2.0 * rows2 * w.N * w.K
    cpu = ""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"rows 0..{rows2 - 1} of the 8192^3 bf16 product ({rows2}x8192 outputs, "
                      f"full K, fp64), {dt:.1f} s wall on {threads} threads ({cpu})",
            "seconds": dt}


def load_traffic(workload: str):
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    entry = t.get(workload)
    if not entry or entry.get("kernel_hash") != kernel_hash():
        return None
    return entry.get("bytes_per_launch")


def main() -> int:
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); "
              "the product needs no exchange between GPUs and no multi-GPU path is built",
              file=sys.stderr)
        return 2
    import torch

    import tensor_core_matrix_amd as tcm
    from tensor_core_matrix_amd import inputs as inp

    tcm.lib()
    if args.only == "copy":
        ms, gbs = copy_ceiling(torch, args.steps, args.warmup)
        print(f"[bench] copy 1 GiB -> 1 GiB: {ms:.4f} ms/call, {gbs:.1f} GB/s", file=sys.stderr,
              flush=True)
        return 0
    order = [args.only] if args.only else ORDER
    # every workload's inputs on the device before the first timed call
    t0 = time.perf_counter()
    prepared = {name: prepare(name, torch, inp, tcm) for name in order}
    torch.cuda.synchronize()
    print(f"[bench] inputs of {len(order)} workloads resident in "
          f"{time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)
    sampler = ClockSampler(torch)
    results = {}
    for name in order:
        pr = prepared[name]
        w = pr.w
        steps = args.steps
        warm = args.warmup if name == ORDER[0] else max(args.warmup, 4 * args.steps)
        if name == "tile_f16":
            steps = max(steps, 200)
        reps = timed(pr.fn, steps, warm, args.repeats, torch)
        # clock and power under sustained calls, after (outside) the timed
        # repeats; the single tile is launch-bound and gets none
        clock = None if name == "tile_f16" or args.no_clock else sampler.window(pr.fn, torch)
        ms = statistics.median(reps)
        tflops = w.flops / (ms * 1e-3) / 1e12
        results[name] = {
            "ms": ms, "tflops": tflops, "steps": steps, "warmup": warm, "repeats": len(reps),
            "repeats_ms": [round(r, 5) for r in reps],
            "frac_of_peak": tflops / PEAK_TFLOPS[w.dtype],
            "gbs": pr.nbytes / (ms * 1e-3) / 1e9, "bytes": pr.nbytes, "sets": pr.sets,
            "clock": clock,
            "plan": tcm.plan(w.M, w.N, w.K, batch=w.batch,
                             mx={"e4m3": 1, "e2m1": 2, "e2m3": 3, "e3m2": 3}.get(w.dtype, 0),
                             dtype=tcm.F16 if w.dtype == "f16" else tcm.BF16,
                             out_dtype=tcm.BF16 if w.out_dtype == "bf16" else tcm.F32,
                             num_cus=0),
        }
        sclk = clock["sclk_mhz"] if clock else None
        print(f"[bench] {name}: {ms:.4f} ms/call (median of {len(reps)} x {steps}), "
              f"{tflops:.1f} TFLOP/s, sclk {sclk} MHz", file=sys.stderr, flush=True)
    del prepared
    torch.cuda.empty_cache()
    copy_ms, copy_gbs = (None, None) if args.only else copy_ceiling(torch)
    if copy_gbs:
        print(f"[bench] copy 1 GiB: {copy_gbs:.1f} GB/s", file=sys.stderr, flush=True)

    head = order[0]
    hw = inp.WORKLOADS[head]
    r = results[head]
    bound = "hbm" if head == "batched" else "mfma"
    if bound == "mfma":
        roof = {"bound": "mfma", "achieved": r["tflops"], "peak": PEAK_TFLOPS[hw.dtype],
                "unit": "TFLOP/s", "frac": r["frac_of_peak"], "traffic": load_traffic(head)}
    else:
        roof = {"bound": "hbm", "achieved": r["gbs"], "peak": HBM_GBS, "unit": "GB/s",
                "frac": r["gbs"] / HBM_GBS, "traffic": load_traffic(head)}
    line = {
        "metric": METRIC,
        "value": r["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": r["steps"],
        "warmup": args.warmup,
        "ms_per_step": r["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": hw.dtype if hw.dtype in ("e4m3", "e2m1", "e2m3", "e3m2") else "bf16",
        "data": "synthetic",
        "config": {"workload": f"{head}: M=N=K={hw.M} TN, {hw.dtype} in, fp32 accumulate, "
                               f"{hw.out_dtype} out, seed {hw.seed}",
                   "tile": [r["plan"]["tile_m"], r["plan"]["tile_n"], r["plan"]["tile_k"]],
                   "stages": r["plan"]["stages"], "grid": r["plan"]["grid"],
                   "repeats": args.repeats, "timing": "median of repeats",
                   "parallelism": "single GPU"},
        "roofline": roof,
        "clock": r["clock"],
        "hbm_copy_gbs": copy_gbs,
        "workloads": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv)
                          for kk, vv in v.items() if kk != "plan"} for k, v in results.items()},
    }
    if not args.no_cpu and not args.only:
        print("[bench] timing the fp64 oracle on the host", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
