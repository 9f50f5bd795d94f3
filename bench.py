"""Benchmark of the MX quantization hot path on one MI355X.

Prints ONE JSON line.  The headline workload is the dual-orientation MXFP8
quantization of a BF16 8192 x 4096 activation (hidden size 4096, sequence 8192):
E4M3 codes along rows and along columns from one read, k = 32 blocks, the
overflow-safe round-up scale rule and the fused per-tensor amax.  A step is one
call of ``mx_quantize_dual`` on a fresh input buffer (8 buffer sets of 130 MiB
rotate, so the 256 MiB last-level cache cannot serve a step from the previous
one); inputs are resident in HBM before the timed region.

``value`` = algorithmic bytes per step (input read + codes, scales and amax
written) x steps / wall time of the timed region.  ``roofline.achieved`` = the
same bytes / the kernel's own average duration (one HIP event pair around the K
back-to-back launches on the stream the kernel runs on).  A second pass brackets
every launch with its own events for the median and the 10th / 90th
percentiles; the graphics clock is polled through the management library while
the kernel runs back to back (and, for long kernels, derived from the committed
rocprofv3 summary's cycle counter); a plain
device copy of the same size gives the attainable copy roof.  The MXFP8 GEMM
(8192 x 4096 x 14336) and the other workloads are reported under ``gemm`` and
``extra``; the CPU oracle under ``cpu_baseline``.

Usage: python bench.py [--gpus 1] [--steps 1000] [--warmup 500] [--no-cpu-baseline] [--no-extra]
       python bench.py --mode dual|delayed|delayed_grad|delayed_small|col|sr|fp6dual|gemm|copy ...
           (one workload only, for profiler passes; 'copy' is a plain 256 MiB
            device copy used to calibrate the byte counters)
       python bench.py --summarize OUT.md --stats S.csv --fetch F.csv --write W.csv
                       --copy-fetch CF.csv --copy-write CW.csv --workload W --kernel K --command "..."
                       [--pmc P.csv ...]
           (turns rocprofv3 outputs into a committed profile summary)
       python bench.py --summarize-gemm profiles --stats S.csv [--pmc-gemm P.csv ...] --command "..."
           (the same for the GEMM kernels)
"""

import argparse
import hashlib
import re
import json
import os
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
FP8_PEAK_TFLOPS = 5000.0         # dense FP8 / MXFP8 MFMA
FP4_PEAK_TFLOPS = 10100.0        # dense MXFP4 MFMA
FP6_PEAK_TFLOPS = 10100.0        # dense MXFP6 MFMA
METRIC = "MX quantize GB/s (% HBM peak); MXFP8 GEMM TFLOP/s (% FP8 MFMA peak)"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "dual_bf16_kernel_mxfp8_bf16_8192x4096.md")
QUANT_SOURCES = ("quantize.hip", "mx_device.hpp")
GEMM_SOURCES = ("gemm.hip", "mx_device.hpp")


def code_digest(texts) -> str:
    """Hash of C++ source texts with comments and blank space removed, so that a
    comment-only edit keeps a counter summary valid and any code edit voids it."""
    h = hashlib.sha256()
    for text in texts:
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def kernel_source_hash(files=QUANT_SOURCES) -> str:
    texts = []
    for f in files:
        with open(os.path.join(ROOT, "mx_block_scaled_quantize_amd", "csrc", f)) as fh:
            texts.append(fh.read())
    return code_digest(texts)


def profile_fields(path):
    """key: value lines of a committed profile summary."""
    vals = {}
    if os.path.exists(path):
        for line in open(path):
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    return vals


def profile_is_current(path, files) -> bool:
    """True when the summary was taken on the kernel source as it stands."""
    return profile_fields(path).get("kernel_source_hash") == kernel_source_hash(files)


def measured_traffic():
    """HBM bytes per dual-quantize launch from the committed rocprofv3 counter
    summary, or None if absent or taken on a different kernel source."""
    vals = profile_fields(TRAFFIC_FILE)
    if vals.get("kernel_source_hash") != kernel_source_hash() or "traffic_bytes_per_launch" not in vals:
        return None
    return float(vals["traffic_bytes_per_launch"].split()[0])


def profile_clock(path, files):
    """GPU clock during a kernel from a committed rocprofv3 summary (GRBM_GUI_ACTIVE
    cycles per XCD over the kernel's duration), when it was taken on the current
    source: the graphics clock a short kernel actually ran at, which a
    management-library sample between launches does not see."""
    vals = profile_fields(path)
    if "gpu_clock_GHz_from_GRBM" not in vals:
        return None
    return {"GHz": float(vals["gpu_clock_GHz_from_GRBM"]), "source": os.path.relpath(path, ROOT),
            "current": vals.get("kernel_source_hash") == kernel_source_hash(files)}


def pct(v, q):
    """q-th percentile (nearest rank) of a sorted list."""
    return v[min(len(v) - 1, max(0, int(round(q / 100.0 * (len(v) - 1)))))]


def launch_distribution(fn, n, stream, torch):
    """Per-launch durations: every launch bracketed by its own event pair."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for s, e in evs:
        s.record(stream)
        fn()
        e.record(stream)
    torch.cuda.synchronize()
    us = sorted(s.elapsed_time(e) * 1e3 for s, e in evs)
    return {"median_us": round(pct(us, 50), 2), "p10_us": round(pct(us, 10), 2), "p90_us": round(pct(us, 90), 2),
            "min_us": round(us[0], 2), "max_us": round(us[-1], 2), "launches": n}


def clock_under_load(fn, dev, torch, seconds=2.0, settle=1.0, burst=50):
    """Graphics clock while fn's kernel runs back to back: the management library's
    current GFX clock and GFX activity (amdsmi), polled from a thread every 10 ms
    after `settle` seconds of a `seconds`-long run of bursts of launches on the
    device (found by its PCI address).  The library refreshes these figures only
    about once or twice a second, hence the long run and the settling time.  A
    missing library or device gives an "error" entry instead of figures."""
    try:
        import amdsmi
        amdsmi.amdsmi_init()
    except Exception as e:   # no library, or no access to the device's management interface
        return {"MHz_median": None, "error": type(e).__name__}
    try:
        p = torch.cuda.get_device_properties(dev)
        bdf = f"{p.pci_domain_id:04x}:{p.pci_bus_id:02x}:{p.pci_device_id:02x}.0"
        h = amdsmi.amdsmi_get_processor_handle_from_bdf(bdf)
        clk, act, stop = [], [], threading.Event()

        def poll():
            t_start = time.perf_counter() + settle
            while not stop.is_set():
                if time.perf_counter() >= t_start:
                    try:
                        clk.append(int(amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.GFX)["clk"]))
                        a = amdsmi.amdsmi_get_gpu_metrics_info(h).get("average_gfx_activity")
                        if isinstance(a, (int, float)):
                            act.append(a)
                    except Exception:
                        pass
                time.sleep(0.01)

        th = threading.Thread(target=poll, daemon=True)
        torch.cuda.synchronize()
        th.start()
        t_end = time.perf_counter() + seconds
        while time.perf_counter() < t_end:
            for _ in range(burst):
                fn()
            torch.cuda.synchronize()
        stop.set()
        th.join()
        if not clk:
            return {"MHz_median": None, "error": "no samples", "bdf": bdf}
        clk.sort()
        act.sort()
        return {"MHz_median": pct(clk, 50), "MHz_min": clk[0], "MHz_max": clk[-1], "samples": len(clk),
                "gfx_activity_pct_median": pct(act, 50) if act else None, "bdf": bdf,
                "source": f"amdsmi GFX clock, polled over the last {seconds - settle:.1f} s of {seconds:.1f} s "
                          "of back-to-back launches"}
    except Exception as e:
        return {"MHz_median": None, "error": type(e).__name__}
    finally:
        try:
            amdsmi.amdsmi_shut_down()
        except Exception:
            pass


def copy_roof(torch, dev, stream, nbytes=64 << 20, sets=8, n=50):
    """A plain device copy of nbytes (read nbytes, write nbytes) through rotating
    buffer sets: the attainable streaming rate at this size."""
    bufs = [(torch.ones(nbytes, dtype=torch.uint8, device=dev), torch.empty(nbytes, dtype=torch.uint8, device=dev))
            for _ in range(sets)]
    idx = [0]

    def fn():
        s, d = bufs[idx[0] % sets]
        d.copy_(s)
        idx[0] += 1
    t = time_calls(fn, n, 5, stream, torch)
    del bufs
    return {"GB/s": round(2 * nbytes / t / 1e9, 1), "us": round(t * 1e6, 2), "bytes_read": nbytes,
            "bytes_written": nbytes, "frac_of_spec": round(2 * nbytes / t / 1e9 / HBM_PEAK_GBS, 4),
            "kind": "torch device-to-device copy_, 8 rotating buffer sets"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # 500 warm-up launches after the clock probe, 1000 timed (about 45 ms): with 5 and
    # 200 the first launches after the probe, still slower, raised the average by 5%
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--mode", choices=["full", "dual", "delayed", "delayed_grad", "delayed_small", "col", "sr",
                                       "fp6dual", "gemm",
                                       "copy"], default="full")
    ap.add_argument("--workload", default="dual", help="which workload --summarize describes")
    ap.add_argument("--summarize", metavar="OUT_MD")
    ap.add_argument("--summarize-gemm", metavar="OUT_DIR")
    ap.add_argument("--pmc-gemm", nargs="*", default=[])
    ap.add_argument("--pmc", nargs="*", default=[])
    ap.add_argument("--stats")
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--copy-fetch")
    ap.add_argument("--copy-write")
    ap.add_argument("--command", default="")
    ap.add_argument("--kernel", default="dual_bf16_kernel<0, 1, true>")
    args = ap.parse_args()
    if args.summarize_gemm:
        summarize_gemm(args)
        return
    if args.summarize:
        summarize(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the quantizers and the GEMM run on a single "
              "MI355X here (multi-GPU sharding is described, not built); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import mx_block_scaled_quantize_amd as mxa
    import workloads

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    lib = mxa.lib
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream

    def up_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    if args.mode == "copy":
        n = 256 << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        t = time_calls(lambda: dst.copy_(src), args.steps, args.warmup, stream, torch)
        print(json.dumps({"mode": "copy", "bytes_read": n, "bytes_written": n, "us": round(t * 1e6, 2),
                          "GB/s": round(2 * n / t / 1e9, 1)}), flush=True)
        return
    if args.mode == "delayed_small":   # the per-call cost of a launch-bound delayed-scaling call only
        res = bench_delayed(lib, sp, stream, dev, up_bf16, mxa, workloads, torch, streams=(), with_null=False)
        print(json.dumps({"mode": args.mode, **res}), flush=True)
        return
    if args.mode in ("delayed", "delayed_grad"):
        res = bench_delayed(lib, sp, stream, dev, up_bf16, mxa, workloads, torch, args.steps,
                            streams=("act",) if args.mode == "delayed" else ("grad",), with_null=False,
                            with_small=False)
        print(json.dumps({"mode": args.mode, **res}), flush=True)
        return
    if args.mode in ("col", "sr", "fp6dual"):
        res = {"col": bench_wgrad_quant, "sr": bench_sr, "fp6dual": bench_fp6}[args.mode](
            lib, sp, stream, dev, up_bf16, mxa, workloads, np, torch, args.steps)
        print(json.dumps({"mode": args.mode, **res}), flush=True)
        return
    if args.mode == "gemm":
        print(json.dumps({"mode": "gemm", "gemm": bench_gemm(lib, sp, stream, dev, up_bf16, mxa, workloads, np,
                                                             torch, args.steps),
                          "gemm_fp4": bench_gemm_fp4(lib, sp, stream, dev, up_bf16, workloads, torch, args.steps),
                          "mm_fp8": bench_mm_fp8(lib, sp, stream, dev, up_bf16, mxa, workloads, torch, args.steps),
                          "requant": bench_gemm_requant(lib, sp, stream, dev, up_bf16, mxa, workloads, torch,
                                                        args.steps),
                          "gemm_fp6": bench_gemm_fp6(lib, sp, stream, dev, up_bf16, mxa, workloads, torch,
                                                     args.steps)}),
              flush=True)
        return

    # ------------------------------------------------------------------ headline: dual quantize
    R, C = 8192, 4096
    algo_bytes = R * C * 2 + 2 * R * C + 2 * (R * C // 32) + 4      # 136,314,884
    x0 = up_bf16(workloads.activation_bf16())
    nsets = 8
    sets = []
    for i in range(nsets):
        x = x0 if i == 0 else x0.clone()
        sets.append(dict(x=x,
                         qr=torch.empty((R, C), dtype=torch.uint8, device=dev),
                         sr=torch.empty((R, C // 32), dtype=torch.uint8, device=dev),
                         qc=torch.empty((C, R), dtype=torch.uint8, device=dev),
                         sc=torch.empty((C, R // 32), dtype=torch.uint8, device=dev),
                         a=torch.zeros(1, dtype=torch.float32, device=dev)))
    idx = [0]

    # the call's arguments per buffer set, built once: the per-launch host work (a
    # ctypes call and HIP's launch) must stay below the kernel's ~28 us, or the
    # event timing measures the host loop rather than the kernel
    dual_fn = lib.mx_quantize_dual
    dual_args = [(s["x"].data_ptr(), 1, R, C, 32, 0, 1, s["qr"].data_ptr(), s["sr"].data_ptr(), s["qc"].data_ptr(),
                  s["sc"].data_ptr(), 0, s["a"].data_ptr(), sp) for s in sets]

    def dual():
        i = idx[0]
        idx[0] = i + 1
        st = dual_fn(*dual_args[i % nsets])
        if st != 0:
            raise RuntimeError(lib.mx_status_str(st).decode())

    # the graphics clock under this load: two seconds of the same launches, before
    # the warm-up, so that the timed region starts on a GPU out of its idle state
    # (a fresh box otherwise spends the first milliseconds ramping up, longer than
    # a short timed region)
    clock = clock_under_load(dual, dev, torch)
    for i in range(args.warmup):
        dual()
    torch.cuda.synchronize()
    # one event pair around the K back-to-back launches on the kernel's stream:
    # their average is the kernel's average launch duration (no per-launch
    # event overhead inside the region)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        dual()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dist = launch_distribution(dual, max(args.steps, 50), stream, torch)
    avg_kern_s = e0.elapsed_time(e1) / args.steps / 1e3
    ms_per_step = wall / args.steps * 1e3
    value = algo_bytes * args.steps / wall / 1e9
    achieved = algo_bytes / avg_kern_s / 1e9
    traffic = measured_traffic()
    del sets
    roof = copy_roof(torch, dev, stream)

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "MXFP8 E4M3 dual (row + column, one read) quantization of a BF16 8192x4096 "
                               "activation, k=32, round-up E8M0 scale, fused per-tensor amax",
                   "rows": R, "cols": C, "in_dtype": "bf16", "element": "e4m3", "scale_rule": "ceil",
                   "bytes_per_step": algo_bytes, "buffer_sets": nsets},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else round(traffic)},
        "kernel_us": round(avg_kern_s * 1e6, 2),
        "launch_us": dist,
        "gpu_clock": {"under_load": clock, "profile": profile_clock(TRAFFIC_FILE, QUANT_SOURCES)},
        "copy_roof": roof,
        "frac_of_copy_roof": round(achieved / roof["GB/s"], 4),
    }

    # ------------------------------------------------------------------ GEMM + other workloads
    if args.mode == "dual":
        print(json.dumps(out), flush=True)
        return
    if not args.no_extra:
        out["gemm"] = bench_gemm(lib, sp, stream, dev, up_bf16, mxa, workloads, np, torch)
        out["extra"] = bench_extra(lib, sp, stream, dev, up_bf16, mxa, workloads, np, torch)

    # ------------------------------------------------------------------ CPU oracle baseline
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(workloads, np)

    print(json.dumps(out), flush=True)


def time_calls(fn, n, warm, stream, torch):
    """Average duration of fn's launches: one event pair around n back-to-back calls."""
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(n):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n / 1e3


def time_alternating(fns, n, rounds, stream, torch, warm=2):
    """Average launch durations of several variants measured in alternation
    (A B A B ...), so that a drift of the clock under load does not favour the
    variant measured first: {name: mean over the rounds of time_calls}."""
    acc = {k: 0.0 for k in fns}
    for r in range(rounds):
        for k, fn in fns.items():
            acc[k] += time_calls(fn, n, warm if r == 0 else 0, stream, torch)
    return {k: v / rounds for k, v in acc.items()}


# GEMM legs: the first launches of a burst run while the clock is still settling
# (their durations drift by up to 20% over the first 30 to 40 calls of an 8192 x
# 14336 x 4096 GEMM, about 15 ms), so each leg is warmed up with GEMM_WARM calls
# and timed over at least GEMM_CALLS.
GEMM_WARM, GEMM_CALLS = 40, 20


def gemm_calls(steps):
    return max(steps, GEMM_CALLS)


# Memory-bound legs rotate through enough buffer sets that one call's data is
# long gone from the 256 MiB last-level cache when it comes round again.
CACHE_DEFEAT_BYTES = 768 << 20
# ... and are warmed up with at least HBM_WARM launches and timed over at least
# HBM_CALLS (a multiple of 32: whole 32-step delayed-scaling sequences): the
# first launches after a pause run slower (5% on the dual after 5 warm-up launches).
HBM_WARM, HBM_CALLS = 300, 320


def time_rotating(make_set, call, per_call_bytes, n, warm, stream, torch, dist=False):
    """time_calls over ceil(768 MiB / per_call_bytes) (2..16) buffer sets used in turn,
    with at least HBM_WARM warm-up and HBM_CALLS timed launches; with dist, also the
    per-launch distribution of n launches."""
    k = max(2, min(16, -(-CACHE_DEFEAT_BYTES // per_call_bytes)))
    sets = [make_set(i) for i in range(k)]
    idx = [0]

    def fn():
        call(sets[idx[0] % k], idx[0])
        idx[0] += 1
    t = time_calls(fn, max(n, HBM_CALLS), max(warm, HBM_WARM), stream, torch)
    d = launch_distribution(fn, n, stream, torch) if dist else None
    del sets
    return (t, k, d) if dist else (t, k)


def hbm_leg(t, nbytes, k, dist=None):
    r = {"us": round(t * 1e6, 2), "GB/s": round(nbytes / t / 1e9, 1),
         "hbm_frac": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4), "bytes_per_call": nbytes, "buffer_sets": k}
    if dist:
        r["launch_us"] = dist
    return r


def bench_delayed(lib, sp, stream, dev, up_bf16, mxa, workloads, torch, steps=32, streams=("act", "grad"),
                  with_null=True, with_small=True):
    """Per-tensor delayed scaling, BF16 8192 x 4096 -> transposed FP8 with the ring
    fold: the activation stream (E4M3) and the gradient stream (E5M2), each on its
    own ring of 16 with ticket scratch; the activation stream also on the page's
    plain ring without scratch; and the per-call cost on a small 128 x 256 tensor,
    where the call is launch-bound (the fixed overhead per linear layer)."""
    R, C = 8192, 4096
    b3 = R * C * 2 + R * C + 80
    res = {}
    for stream_name in streams:
        fmt = {"act": 0, "grad": 1}[stream_name]
        fp8_max = workloads.DELAYED_FP8_MAX[stream_name]
        xs = [up_bf16(workloads.delayed_step(stream_name, t)) for t in range(2)]
        modes = (("scratch", True), ("no_scratch", False)) if with_null and stream_name == "act" else \
            (("scratch", True),)
        for mode, use_scratch in modes:
            ring = mxa.new_ring(16, dev)
            tickets = mxa.new_tickets(dev) if use_scratch else None

            def d_set(i):
                return dict(x=xs[i % 2] if i < 2 else xs[i % 2].clone(),
                            qT=torch.empty((C, R), dtype=torch.uint8, device=dev))

            def delayed(st, t):
                mxa.check(lib.fp8_quantize_delayed(st["x"].data_ptr(), 1, R, C, fmt, 1, None, st["qT"].data_ptr(),
                                                   ring.data_ptr(), 16, t % 16, fp8_max, 1.0, None,
                                                   None if tickets is None else tickets.data_ptr(), sp))
            t3, k3, d3 = time_rotating(d_set, delayed, b3, steps, 4, stream, torch, dist=True)
            name = f"delayed_fp8_{mxa_fmt(fmt)}_transposed_bf16_8192x4096" + ("" if use_scratch else "_no_scratch")
            res[name] = hbm_leg(t3, b3, k3, d3)
        del xs
    if not with_small:
        return res
    # per-call fixed cost: a launch-bound 128 x 256 call, ring fold included
    x = up_bf16(workloads.delayed_step("act", 0, rows=128, cols=256))
    qT = torch.empty((256, 128), dtype=torch.uint8, device=dev)
    ring = mxa.new_ring(16, dev)
    tickets = mxa.new_tickets(dev)
    n = 200
    calls = [0]

    def small():
        mxa.check(lib.fp8_quantize_delayed(x.data_ptr(), 1, 128, 256, 0, 1, None, qT.data_ptr(), ring.data_ptr(), 16,
                                           calls[0] % 16, 448.0, 1.0, None, tickets.data_ptr(), sp))
        calls[0] += 1
    for _ in range(10):
        small()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    h0 = time.perf_counter()
    e0.record(stream)
    for _ in range(n):
        small()
    h1 = time.perf_counter()
    e1.record(stream)
    torch.cuda.synchronize()
    res["delayed_fp8_e4m3_transposed_bf16_128x256_per_call"] = {
        "gpu_us_per_call": round(e0.elapsed_time(e1) / n * 1e3, 2),
        "host_enqueue_us_per_call": round((h1 - h0) / n * 1e6, 2),
        "launch_us": launch_distribution(small, n, stream, torch),
        "note": "back-to-back calls on one stream; the GPU time per call is the fixed cost of a call "
                "(launch, ring fold) on a launch-bound tensor"}
    return res


def mxa_fmt(code):
    return {0: "e4m3", 1: "e5m2"}[code]


def bench_gemm(lib, sp, stream, dev, up_bf16, mxa, workloads, np, torch, steps=10):
    """MXFP8 E4M3 GEMM 8192 x 4096 . (14336 x 4096)^T, BF16 out (quantized operands resident), with the
    operands' scales row-major (the headline figure) and in the GEMM layout ("gemm_scales")."""
    M, N, K = 8192, 14336, 4096
    a_bits, w_bits = workloads.mlp_operands()
    flops = 2.0 * M * N * K
    c = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ops = {layout: (mxa.mx_quantize(up_bf16(a_bits), "e4m3", "ceil", "row", scale_layout=layout),
                    mxa.mx_quantize(up_bf16(w_bits), "e4m3", "ceil", "row", scale_layout=layout))
           for layout in ("row", "gemm")}

    def call(layout):
        (qa, sa), (qw, sw) = ops[layout]
        return lambda: mxa.check(lib.mx_gemm(qa.data_ptr(), sa.data_ptr(), 0, qw.data_ptr(), sw.data_ptr(), 0,
                                             mxa.SCALE_LAYOUT[layout], M, N, K, 1.0, c.data_ptr(), 1, N, sp))
    times = time_alternating({k: call(k) for k in ops}, gemm_calls(steps), 2, stream, torch, warm=GEMM_WARM)
    clock = clock_under_load(call("row"), dev, torch, burst=4)
    del ops
    vendor = vendor_fp8_reference(lib, sp, stream, dev, up_bf16, workloads, torch, c, steps)
    t = times["row"]
    tf = flops / t / 1e12
    prof = os.path.join(ROOT, "profiles", "gemm256_kernel_mxfp8_8192x14336x4096.md")
    return {"workload": "MXFP8 E4M3 block-scaled GEMM 8192x4096 x (14336x4096)^T, FP32 accumulate, BF16 out",
            "value": round(tf, 1), "unit": "TFLOP/s", "ms_per_call": round(t * 1e3, 4),
            "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / FP8_PEAK_TFLOPS, 4), "traffic": None},
            "gemm_scales": {"ms_per_call": round(times["gemm"] * 1e3, 4),
                            "TFLOP/s": round(flops / times["gemm"] / 1e12, 1),
                            "frac": round(flops / times["gemm"] / 1e12 / FP8_PEAK_TFLOPS, 4)},
            "profile": {"file": os.path.relpath(prof, ROOT), "current": profile_is_current(prof, GEMM_SOURCES)},
            "gpu_clock": {"under_load": clock, "profile": profile_clock(prof, GEMM_SOURCES)},
            "vendor_reference": vendor}


def vendor_fp8_reference(lib, sp, stream, dev, up_bf16, workloads, torch, c, steps):
    """Context only, not this library's figure: the vendor BLAS's per-tensor FP8 GEMM
    (torch._scaled_mm, served by hipBLASLt) on the same shape and box, timed in
    alternation with this library's per-tensor mm_fp8 on the same FP8 operands."""
    M, N, K = 8192, 14336, 4096
    a_bits, w_bits = workloads.mlp_operands()
    try:
        x, w = up_bf16(a_bits), up_bf16(w_bits)
        sx = (x.float().abs().max() / 448).reshape(())
        sw = (w.float().abs().max() / 448).reshape(())
        x8 = (x.float() / sx).to(torch.float8_e4m3fn)
        w8 = (w.float() / sw).to(torch.float8_e4m3fn)
        del x, w
        scale = (sx * sw).reshape(1).contiguous()

        def ours():
            st = lib.mm_fp8(x8.data_ptr(), w8.data_ptr(), 0, 1, M, N, K, 0, 0, 0, 1, scale.data_ptr(), None,
                            c.data_ptr(), sp)
            if st != 0:
                raise RuntimeError(lib.mx_status_str(st).decode())

        def vendor():
            torch._scaled_mm(x8, w8.t(), scale_a=sx.float(), scale_b=sw.float(), out_dtype=torch.bfloat16)

        times = time_alternating({"ours": ours, "vendor": vendor}, gemm_calls(steps), 2, stream, torch,
                                 warm=GEMM_WARM)
    except Exception as e:   # an FP8 GEMM the installed torch cannot run here
        return {"error": f"{type(e).__name__}: {str(e)[:120]}"}
    flops = 2.0 * M * N * K
    return {"what": "per-tensor FP8 E4M3 GEMM 8192x4096 x (14336x4096)^T, BF16 out: torch._scaled_mm (hipBLASLt) "
                    "against this library's mm_fp8, in alternation; context only",
            "vendor_ms_per_call": round(times["vendor"] * 1e3, 4),
            "vendor_frac": round(flops / times["vendor"] / 1e12 / FP8_PEAK_TFLOPS, 4),
            "mm_fp8_ms_per_call": round(times["ours"] * 1e3, 4),
            "mm_fp8_frac": round(flops / times["ours"] / 1e12 / FP8_PEAK_TFLOPS, 4)}


def bench_extra(lib, sp, stream, dev, up_bf16, mxa, workloads, np, torch):
    res = {}
    # row-wise quantize + dequantize, FP32 256 x 1024, round-down rule
    x = torch.from_numpy(workloads.wide_range_f32()).to(dev)
    q = torch.empty((256, 1024), dtype=torch.uint8, device=dev)
    s = torch.empty((256, 32), dtype=torch.uint8, device=dev)
    d = torch.empty((256, 1024), dtype=torch.float32, device=dev)
    tq = time_calls(lambda: lib.mx_quantize(x.data_ptr(), 0, 256, 1024, 32, 0, 0, 0, 0, 0, q.data_ptr(),
                                            s.data_ptr(), 0, None, sp), 50, 5, stream, torch)
    td = time_calls(lambda: lib.mx_dequantize(q.data_ptr(), s.data_ptr(), 256, 1024, 32, 0, 0, 0, d.data_ptr(), 0,
                                              sp), 50, 5, stream, torch)
    b1 = 256 * 1024 * 4 + 256 * 1024 + 256 * 32
    res["rowwise_quant_f32_256x1024"] = {"us": round(tq * 1e6, 2), "GB/s": round(b1 / tq / 1e9, 1)}
    res["dequant_f32_256x1024"] = {"us": round(td * 1e6, 2), "GB/s": round(b1 / td / 1e9, 1)}
    res.update(bench_delayed(lib, sp, stream, dev, up_bf16, mxa, workloads, torch))
    res.update(bench_sr(lib, sp, stream, dev, up_bf16, mxa, workloads, np, torch))
    res.update(bench_fp6(lib, sp, stream, dev, up_bf16, mxa, workloads, np, torch))
    res.update(bench_wgrad_quant(lib, sp, stream, dev, up_bf16, mxa, workloads, np, torch))
    g_bits, x_bits, mask = workloads.weight_grad_operands()
    st0 = wgrad_set(dev, up_bf16(g_bits), up_bf16(x_bits), torch)
    st1 = wgrad_set(dev, st0["G"], st0["X"], torch)
    wgrad_quant(lib, sp, mxa, st0, mask, 0)
    wgrad_quant(lib, sp, mxa, st1, mask, 1)
    res.update(time_gemm_fp4_layouts(lib, sp, stream, dev, st0, st1, torch, 10))
    del st0, st1
    res.update(bench_mm_fp8(lib, sp, stream, dev, up_bf16, mxa, workloads, torch))
    res.update(bench_gemm_requant(lib, sp, stream, dev, up_bf16, mxa, workloads, torch))
    res.update(bench_gemm_fp6(lib, sp, stream, dev, up_bf16, mxa, workloads, torch))
    return res


def bench_sr(lib, sp, stream, dev, up_bf16, mxa, workloads, np, torch, steps=32):
    """Stochastic-rounding MXFP4 row-wise of a BF16 8192 x 4096 gradient, one uint32 word per element."""
    R, C = 8192, 4096
    gx = up_bf16(workloads.activation_bf16(R, C))
    words = torch.from_numpy(workloads.random_words((R, C), 47).view(np.int32)).to(dev)
    bsr = R * C * 2 + R * C * 4 + R * C // 2 + R * C // 32

    def sr_set(i):
        return dict(x=gx if i == 0 else gx.clone(), w=words if i == 0 else words.clone(),
                    q=torch.empty((R, C // 2), dtype=torch.uint8, device=dev),
                    s=torch.empty((R, C // 32), dtype=torch.uint8, device=dev))
    t, k, d = time_rotating(sr_set, lambda st, i: mxa.check(lib.mx_quantize_sr(
        st["x"].data_ptr(), 1, R, C, 32, 2, 1, st["w"].data_ptr(), st["q"].data_ptr(), st["s"].data_ptr(), None, sp)),
        bsr, steps, 4, stream, torch, dist=True)
    return {"sr_mxfp4_rowwise_bf16_8192x4096": hbm_leg(t, bsr, k, d)}


def bench_fp6(lib, sp, stream, dev, up_bf16, mxa, workloads, np, torch, steps=32):
    """MXFP6 E3M2 of a BF16 8192 x 4096 tensor: row-wise, and dual (both orientations from one read)."""
    R, C = 8192, 4096
    gx = up_bf16(workloads.activation_bf16(R, C))
    bf6 = R * C * 2 + R * C * 3 // 4 + R * C // 32

    def f6_set(i):
        return dict(x=gx if i == 0 else gx.clone(), q=torch.empty((R, C * 3 // 4), dtype=torch.uint8, device=dev),
                    s=torch.empty((R, C // 32), dtype=torch.uint8, device=dev),
                    qc=torch.empty((C, R * 3 // 4), dtype=torch.uint8, device=dev),
                    sc=torch.empty((C, R // 32), dtype=torch.uint8, device=dev))
    t, k, d = time_rotating(f6_set, lambda st, i: mxa.check(lib.mx_quantize(
        st["x"].data_ptr(), 1, R, C, 32, 4, 1, 0, 0, 0, st["q"].data_ptr(), st["s"].data_ptr(), 0, None, sp)),
        bf6, steps, 4, stream, torch, dist=True)
    res = {"mxfp6_e3m2_rowwise_bf16_8192x4096": hbm_leg(t, bf6, k, d)}
    bf6d = R * C * 2 + 2 * (R * C * 3 // 4 + R * C // 32)
    t, k, d = time_rotating(f6_set, lambda st, i: mxa.check(lib.mx_quantize_dual(
        st["x"].data_ptr(), 1, R, C, 32, 4, 1, st["q"].data_ptr(), st["s"].data_ptr(), st["qc"].data_ptr(),
        st["sc"].data_ptr(), 0, None, sp)), bf6d, steps, 4, stream, torch, dist=True)
    res["mxfp6_e3m2_dual_bf16_8192x4096"] = hbm_leg(t, bf6d, k, d)
    return res


def wgrad_set(dev, G, X, torch):
    return dict(G=G, X=X, gq=torch.empty((4096, 4096), dtype=torch.uint8, device=dev),
                gs=torch.empty((4096, 256), dtype=torch.uint8, device=dev),
                xq=torch.empty((4096, 4096), dtype=torch.uint8, device=dev),
                xs=torch.empty((4096, 256), dtype=torch.uint8, device=dev))


def wgrad_quant(lib, sp, mxa, st, mask, layout=0):
    """Hadamard + column-wise MXFP4 (round-up rule) of both weight-gradient operands
    (scales row-major, or in the GEMM layout with layout=1)."""
    mxa.check(lib.mx_quantize(st["G"].data_ptr(), 1, 8192, 4096, 32, 2, 1, 1, 1, mask, st["gq"].data_ptr(),
                              st["gs"].data_ptr(), layout, None, sp))
    mxa.check(lib.mx_quantize(st["X"].data_ptr(), 1, 8192, 4096, 32, 2, 1, 1, 1, mask, st["xq"].data_ptr(),
                              st["xs"].data_ptr(), layout, None, sp))


def bench_wgrad_quant(lib, sp, stream, dev, up_bf16, mxa, workloads, np, torch, steps=20):
    """Hadamard + column-wise MXFP4 quantization of both BF16 8192 x 4096 weight-gradient operands."""
    g_bits, x_bits, mask = workloads.weight_grad_operands()
    G, X = up_bf16(g_bits), up_bf16(x_bits)
    b5 = 2 * (8192 * 4096 * 2 + 4096 * 4096 + 4096 * 256)
    t, k, d = time_rotating(lambda i: wgrad_set(dev, G if i == 0 else G.clone(), X if i == 0 else X.clone(), torch),
                            lambda st, i: wgrad_quant(lib, sp, mxa, st, mask), b5, steps, 3, stream, torch, dist=True)
    return {"hadamard_mxfp4_colwise_quant_2x_bf16_8192x4096": hbm_leg(t, b5, k, d)}


def bench_gemm_fp6(lib, sp, stream, dev, up_bf16, mxa, workloads, torch, steps=5):
    """The 8192 x 14336 x 4096 MLP GEMM shape with both operands quantized row-wise to MXFP6 E2M3
    (round-up scale), BF16 out, on the 256 x 256 LDS-DMA path."""
    M, N, K = 8192, 14336, 4096
    a_bits, w_bits = workloads.mlp_operands()
    qa, sa = mxa.mx_quantize(up_bf16(a_bits), "e2m3", "ceil", "row")
    qw, sw = mxa.mx_quantize(up_bf16(w_bits), "e2m3", "ceil", "row")
    c = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    t = time_calls(lambda: mxa.check(lib.mx_gemm(qa.data_ptr(), sa.data_ptr(), 3, qw.data_ptr(), sw.data_ptr(), 3, 0, M, N,
                                                 K, 1.0, c.data_ptr(), 1, N, sp)), gemm_calls(steps), GEMM_WARM,
                   stream, torch)
    f = 2.0 * M * N * K
    return {"mxfp6_e2m3_gemm_8192x14336x4096": {"us": round(t * 1e6, 2), "TFLOP/s": round(f / t / 1e12, 1),
                                                "mfma_frac": round(f / t / 1e12 / FP6_PEAK_TFLOPS, 4)}}


def bench_gemm_requant(lib, sp, stream, dev, up_bf16, mxa, workloads, torch, steps=10):
    """The MXFP8 GEMM 8192 x 4096 . (14336 x 4096)^T with its FP32 result re-quantized to MXFP8 E4M3 (round-up
    scale) in the epilogue: codes [8192][14336] + scales instead of a BF16 matrix."""
    M, N, K = 8192, 14336, 4096
    a_bits, w_bits = workloads.mlp_operands()
    qa, sa = mxa.mx_quantize(up_bf16(a_bits), "e4m3", "ceil", "row")
    qw, sw = mxa.mx_quantize(up_bf16(w_bits), "e4m3", "ceil", "row")
    qc = torch.empty((M, N), dtype=torch.uint8, device=dev)
    sc = torch.empty((M, N // 32), dtype=torch.uint8, device=dev)

    def call():
        mxa.check(lib.mx_gemm_requant(qa.data_ptr(), sa.data_ptr(), 0, qw.data_ptr(), sw.data_ptr(), 0, 0, M, N, K, 1.0,
                                      0, 1, qc.data_ptr(), sc.data_ptr(), None, sp))
    t = time_calls(call, gemm_calls(steps), GEMM_WARM, stream, torch)
    tf = 2.0 * M * N * K / t / 1e12
    return {"mxfp8_gemm_requant_e4m3_8192x14336x4096": {"us": round(t * 1e6, 2), "TFLOP/s": round(tf, 1),
                                                        "mfma_frac": round(tf / FP8_PEAK_TFLOPS, 4)}}


def bench_mm_fp8(lib, sp, stream, dev, up_bf16, mxa, workloads, torch, steps=10):
    """Per-tensor FP8 GEMM (mm_fp8) of the MLP up-projection: x [8192][4096] and
    w [14336][4096] cast by the delayed-scaling FP8 quantizer (its second step, so
    the rings hold real scales), scale = s_x s_w on the device, BF16 bias, BF16 out.
    'nt': w as stored [N][K] (x @ w.t(), K-contiguous); 'nn': its transposed copy
    [K][N] (N-contiguous, read through the LDS transpose)."""
    M, N, K = 8192, 14336, 4096
    a_bits, w_bits = workloads.mlp_operands()
    x, w = up_bf16(a_bits), up_bf16(w_bits)
    rx, rw = mxa.new_ring(16, dev), mxa.new_ring(16, dev)
    for step in range(2):
        xq, _ = mxa.fp8_quantize_delayed(x, rx, step, "e4m3", "row")
        wq, wqT = mxa.fp8_quantize_delayed(w, rw, step, "e4m3", "dual")
    del x, w
    scale = (rx[16:17] * rw[16:17]).contiguous()
    bias = up_bf16(workloads.to_bf16_bits(workloads.rng(4, 2).standard_normal(N) * 0.1))
    c = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    flops = 2.0 * M * N * K
    res = {}
    for name, b, tb in (("nt", wq, 1), ("nn", wqT, 0)):
        def call():
            mxa.check(lib.mm_fp8(xq.data_ptr(), b.data_ptr(), 0, 1, M, N, K, 0, 0, 0, tb, scale.data_ptr(),
                                 bias.data_ptr(), c.data_ptr(), sp))
        t = time_calls(call, gemm_calls(steps), GEMM_WARM, stream, torch)
        tf = flops / t / 1e12
        res[f"mm_fp8_e4m3_{name}_bias_8192x14336x4096"] = {"us": round(t * 1e6, 2), "TFLOP/s": round(tf, 1),
                                                            "mfma_frac": round(tf / FP8_PEAK_TFLOPS, 4)}
    return res


def time_gemm_fp4_layouts(lib, sp, stream, dev, st_row, st_gemm, torch, steps):
    """The MXFP4 weight-gradient GEMM on row-major scales (st_row) and on GEMM-layout scales
    (st_gemm), measured in alternation."""
    dw = torch.empty((4096, 4096), dtype=torch.bfloat16, device=dev)

    def call(st, layout):
        return lambda: lib.mx_gemm(st["gq"].data_ptr(), st["gs"].data_ptr(), 2, st["xq"].data_ptr(),
                                   st["xs"].data_ptr(), 2, layout, 4096, 4096, 8192, 1.0 / 32, dw.data_ptr(), 1, 4096,
                                   sp)
    t = time_alternating({"row": call(st_row, 0), "gemm": call(st_gemm, 1)}, gemm_calls(steps), 3, stream, torch,
                         warm=GEMM_WARM)
    f = 2.0 * 4096 * 4096 * 8192
    leg = lambda x: {"us": round(x * 1e6, 2), "TFLOP/s": round(f / x / 1e12, 1),   # noqa: E731
                     "mfma_frac": round(f / x / 1e12 / FP4_PEAK_TFLOPS, 4)}
    return {"mxfp4_gemm_4096x4096x8192": leg(t["row"]), "mxfp4_gemm_4096x4096x8192_gemm_scales": leg(t["gemm"])}


def bench_gemm_fp4(lib, sp, stream, dev, up_bf16, workloads, torch, steps=10):
    """The MXFP4 weight-gradient GEMM alone, on the Hadamard + MXFP4 column-wise operands, with
    row-major and with GEMM-layout scales."""
    import mx_block_scaled_quantize_amd as mxa
    g_bits, x_bits, mask = workloads.weight_grad_operands()
    st0 = wgrad_set(dev, up_bf16(g_bits), up_bf16(x_bits), torch)
    st1 = wgrad_set(dev, st0["G"], st0["X"], torch)
    wgrad_quant(lib, sp, mxa, st0, mask, 0)
    wgrad_quant(lib, sp, mxa, st1, mask, 1)
    return time_gemm_fp4_layouts(lib, sp, stream, dev, st0, st1, torch, steps)


def _pmc_mean(path, kernel_substr, counter):
    import csv
    vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(path))
            if kernel_substr in r["Kernel_Name"] and r["Counter_Name"] == counter]
    return sum(vals) / len(vals), len(vals)


GEMM_PROFILES = {
    # kernel name substring -> (file, title, FLOPs per launch, dense peak TFLOP/s)
    "gemm256_kernel<0, 0, true, false, false, false, false>": (
        "gemm256_kernel_mxfp8_8192x14336x4096.md", "MXFP8 E4M3 GEMM, A 8192x4096 . (W 14336x4096)^T, BF16 out",
        2.0 * 8192 * 14336 * 4096, FP8_PEAK_TFLOPS),
    "gemm256_kernel<2, 2, true, false, false, false, false>": (
        "gemm256_kernel_mxfp4_4096x4096x8192.md",
        "MXFP4 E2M1 GEMM, dW = (1/32) Gq^T Xq, 4096x4096, K = 8192, BF16 out",
        2.0 * 4096 * 4096 * 8192, FP4_PEAK_TFLOPS),
    "gemm256_kernel<0, 0, true, false, false, false, true>": (
        "gemm256_kernel_mxfp8_requant_e4m3_8192x14336x4096.md",
        "MXFP8 E4M3 GEMM 8192x4096 . (14336x4096)^T, FP32 result re-quantized to MXFP8 E4M3 in the epilogue",
        2.0 * 8192 * 14336 * 4096, FP8_PEAK_TFLOPS),
    "gemm256_kernel<0, 0, true, true, false, false, false>": (
        "gemm256_kernel_mm_fp8_nt_8192x14336x4096.md",
        "per-tensor FP8 E4M3 mm_fp8, x 8192x4096 @ w.t() (w 14336x4096 K-contiguous), BF16 bias, BF16 out",
        2.0 * 8192 * 14336 * 4096, FP8_PEAK_TFLOPS),
    "gemm256_kernel<0, 0, true, true, false, true, false>": (
        "gemm256_kernel_mm_fp8_nn_8192x14336x4096.md",
        "per-tensor FP8 E4M3 mm_fp8, x 8192x4096 @ wT (wT 4096x14336 N-contiguous, LDS transpose reads), BF16 bias",
        2.0 * 8192 * 14336 * 4096, FP8_PEAK_TFLOPS),
    "gemm256_kernel<3, 3, true, false, false, false, false>": (
        "gemm256_kernel_mxfp6_e2m3_8192x14336x4096.md",
        "MXFP6 E2M3 GEMM 8192x4096 . (14336x4096)^T, both operands bit-stream packed, BF16 out",
        2.0 * 8192 * 14336 * 4096, FP6_PEAK_TFLOPS),
}


def _pmc_all(paths, kernel_substr):
    """Mean per dispatch of every counter in the given --pmc CSVs for one kernel."""
    import csv
    acc = {}
    for path in paths:
        for r in csv.DictReader(open(path)):
            if kernel_substr in r["Kernel_Name"]:
                acc.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def _counter_lines(counters, avg_ns):
    """Counter lines of a summary, with the derived figures the counters allow
    (GRBM_GUI_ACTIVE is summed over the 8 XCDs; the SQ_* counters over all SIMDs)."""
    lines = [f"{k}_per_dispatch: {v:.6g}" for k, v in sorted(counters.items())]
    grbm = counters.get("GRBM_GUI_ACTIVE")
    if grbm:
        cyc = grbm / 8
        if "SQ_VALU_MFMA_BUSY_CYCLES" in counters:
            lines.append(f"mfma_busy_fraction: {counters['SQ_VALU_MFMA_BUSY_CYCLES'] / (cyc * 1024):.4f}")
        # a counter pass serializes dispatches and stretches short ones, so the
        # clock estimate is only given for kernels long against that overhead
        if avg_ns >= 200e3:
            lines.append(f"gpu_clock_GHz_from_GRBM: {cyc / avg_ns:.3f}")
    waves = counters.get("SQ_WAVES")
    if waves:
        for k in ("SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_LDS", "SQ_INSTS_VMEM_RD", "SQ_INSTS_VMEM_WR",
                  "SQ_INSTS_MFMA"):
            if k in counters:
                lines.append(f"{k}_per_wave: {counters[k] / waves:.1f}")
    if "SQ_LDS_BANK_CONFLICT" in counters and "SQ_LDS_IDX_ACTIVE" in counters and counters["SQ_LDS_IDX_ACTIVE"]:
        lines.append(f"lds_bank_conflict_per_active_cycle: "
                     f"{counters['SQ_LDS_BANK_CONFLICT'] / counters['SQ_LDS_IDX_ACTIVE']:.4f}")
    return lines


def summarize_gemm(args):
    """Profile summaries of the GEMM kernels from a rocprofv3 --stats CSV (and,
    if given, --pmc CSVs: MFMA busy, GRBM, LDS and wait counters)."""
    import csv
    rows = list(csv.DictReader(open(args.stats)))
    for sub, (fname, title, flops, peak) in GEMM_PROFILES.items():
        st = [r for r in rows if sub in r["Name"]]
        if not st:
            continue
        r = st[0]
        avg = float(r["AverageNs"])
        tf = flops / avg / 1e3
        lines = [f"# {sub} -- {title}", "", f"command: {args.command}", "",
                 f"kernel: {r['Name'][:80]}", f"kernel_calls: {r['Calls']}", f"kernel_avg_ns: {avg:.0f}",
                 f"kernel_min_ns: {float(r['MinNs']):.0f}", f"kernel_max_ns: {float(r['MaxNs']):.0f}",
                 f"flops_per_launch: {flops:.0f}", f"achieved_TFLOPs_at_avg: {tf:.1f}",
                 f"fraction_of_dense_peak_{peak:.0f}: {tf / peak:.4f}"]
        if args.pmc_gemm:
            lines += _counter_lines(_pmc_all(args.pmc_gemm, sub), avg)
        lines.append(f"kernel_source_hash: {kernel_source_hash(GEMM_SOURCES)}")
        lines.append("")
        out = os.path.join(args.summarize_gemm, fname)
        with open(out, "w") as f:
            f.write("\n".join(lines))
        print("\n".join(lines))


R8, C4 = 8192, 4096
WORKLOADS = {
    # --workload -> (title, algorithmic bytes per launch, kernel sources)
    "dual": ("MXFP8 E4M3 dual quantization, BF16 8192x4096, round-up scale, amax",
             R8 * C4 * 2 + 2 * R8 * C4 + 2 * (R8 * C4 // 32) + 4, QUANT_SOURCES),
    "delayed": ("per-tensor delayed-scaling FP8 E4M3 cast, BF16 8192x4096 -> transposed codes, ring of 16",
                R8 * C4 * 2 + R8 * C4 + 80, QUANT_SOURCES),
    "delayed_grad": ("per-tensor delayed-scaling FP8 E5M2 cast (gradient stream), BF16 8192x4096 -> transposed "
                     "codes, ring of 16", R8 * C4 * 2 + R8 * C4 + 80, QUANT_SOURCES),
    "delayed_small": ("per-tensor delayed-scaling FP8 E4M3 cast of a launch-bound BF16 128x256 tensor -> transposed "
                      "codes, ring of 16 (two workgroups, single-level ticket)", 128 * 256 * 2 + 128 * 256 + 80,
                      QUANT_SOURCES),
    "col": ("fixed-sign Hadamard + column-wise MXFP4 E2M1 quantization of one BF16 8192x4096 weight-gradient "
            "operand (8192 tokens), round-up scale", R8 * C4 * 2 + R8 * C4 // 2 + R8 * C4 // 32, QUANT_SOURCES),
    "sr": ("stochastic-rounding MXFP4 row-wise, BF16 8192x4096 + one uint32 word per element",
           R8 * C4 * 6 + R8 * C4 // 2 + R8 * C4 // 32, ("quantize_sr.hip", "mx_device.hpp")),
    "fp6dual": ("MXFP6 E3M2 dual quantization, BF16 8192x4096, round-up scale",
                R8 * C4 * 2 + 2 * (R8 * C4 * 3 // 4 + R8 * C4 // 32), ("quantize_fp6.hip", "mx_device.hpp")),
}


def summarize(args):
    """Write the profile summary of a quantizer kernel from rocprofv3 CSVs.

    FETCH_SIZE / WRITE_SIZE (KiB per dispatch) are scaled by the ratio of the
    known bytes of a plain 256 MiB device copy to what the same counters read
    for it; traffic_bytes_per_launch is their scaled sum."""
    import csv
    title, algo, sources = WORKLOADS[args.workload]
    stats = [r for r in csv.DictReader(open(args.stats)) if args.kernel in r["Name"]]
    avg_ns = float(stats[0]["AverageNs"])
    calls = int(stats[0]["Calls"])
    lines = [f"# {args.kernel} -- {title}", "", f"command: {args.command}", "",
             f"kernel_avg_ns: {avg_ns:.0f}", f"kernel_min_ns: {float(stats[0]['MinNs']):.0f}",
             f"kernel_max_ns: {float(stats[0]['MaxNs']):.0f}", f"kernel_calls: {calls}" +
             ("  (the timed steps, the warm-up and the clock probe: two seconds of the same launches)"
              if args.workload == "dual" else ""),
             f"algorithmic_bytes_per_launch: {algo}", f"achieved_GBps_at_avg: {algo / avg_ns:.1f}",
             f"fraction_of_hbm_peak: {algo / avg_ns / HBM_PEAK_GBS:.4f}"]
    if args.fetch and args.write and args.copy_fetch and args.copy_write:
        copy_bytes_kib = 256 * 1024
        ck = "copyBuffer" if "copyBuffer" in open(args.copy_fetch).read() else "elementwise"
        cf, _ = _pmc_mean(args.copy_fetch, ck, "FETCH_SIZE")
        cw, _ = _pmc_mean(args.copy_write, ck, "WRITE_SIZE")
        kf, nf = _pmc_mean(args.fetch, args.kernel, "FETCH_SIZE")
        kw, nw = _pmc_mean(args.write, args.kernel, "WRITE_SIZE")
        f_scale, w_scale = copy_bytes_kib / cf, copy_bytes_kib / cw
        fetch_b = kf * f_scale * 1024
        write_b = kw * w_scale * 1024
        lines += [f"FETCH_SIZE_KiB_per_dispatch_raw: {kf:.1f}  (n={nf})",
                  f"WRITE_SIZE_KiB_per_dispatch_raw: {kw:.1f}  (n={nw})",
                  f"copy_calibration: 256 MiB copy reads FETCH_SIZE {cf:.1f} KiB, WRITE_SIZE {cw:.1f} KiB "
                  f"-> scale fetch x{f_scale:.4f}, write x{w_scale:.4f}",
                  f"hbm_fetch_bytes_per_launch: {fetch_b:.0f}", f"hbm_write_bytes_per_launch: {write_b:.0f}",
                  f"traffic_bytes_per_launch: {fetch_b + write_b:.0f}",
                  f"traffic_over_algorithmic: {(fetch_b + write_b) / algo:.4f}"]
    if args.pmc:
        lines += _counter_lines(_pmc_all(args.pmc, args.kernel), avg_ns)
    lines += [f"kernel_source_hash: {kernel_source_hash(sources)}", ""]
    with open(args.summarize, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


def cpu_info():
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"cpu_model": model, "os_cpu_count": os.cpu_count()}


def _grow(run, nbytes_of, first, full, target_s):
    """Run `run(n)` on growing leading samples (first, 2 first, ...) until about
    target_s seconds were spent or the whole input was done; the rate of the
    largest sample: (n, seconds, GB/s)."""
    n, spent = first, 0.0
    while True:
        t0 = time.perf_counter()
        run(n)
        dt = time.perf_counter() - t0
        spent += dt
        if n >= full or spent + 2 * dt > target_s:
            return n, dt, nbytes_of(n) / dt / 1e9, spent
        n = min(full, 2 * n)


def cpu_baseline(workloads, np, target_s=8.0):
    """The CPU oracle as it stands, on bounded samples of the same workloads, on
    the host of the GPU: the headline (dual E4M3 quantization + amax of leading
    row strips of the BF16 8192 x 4096 input, one thread) and, under ``legs``,
    the delayed-scaling cast with its fold, the Hadamard + MXFP4 column-wise
    quantizer (one thread each) and the float64 GEMM reference of the MXFP8 MLP
    product (BLAS, thread count stated)."""
    from oracle import delayed as odl
    from oracle import gemm as og
    from oracle import mx as omx
    cols = 4096
    xb_all = workloads.activation_bf16()

    def dual(rows):
        xs = workloads.bf16_to_f32(xb_all[:rows])
        omx.quantize_dual(xs, "e4m3", "ceil")
        omx.tensor_amax(xs)
    dual_bytes = lambda r: r * cols * 2 + 2 * r * cols + 2 * (r * cols // 32) + 4  # noqa: E731
    rows, dt, rate, spent = _grow(dual, dual_bytes, 256, 8192, target_s)
    out = {"value": round(rate, 6), "unit": "GB/s", "cores": 1, "kind": "oracle",
           "sample": f"first {rows} of 8192 rows of the BF16 8192x4096 input (dual E4M3 quantization + amax), "
                     f"{dt:.1f} s for that strip, {spent:.1f} s of oracle work in total on the host CPU",
           **cpu_info(), "legs": {}}
    del xb_all
    # delayed scaling: cast with the ring's multiplier + amax + fold, leading rows of step 0
    xd = workloads.bf16_to_f32(workloads.delayed_step("act", 0))

    def delayed(r):
        odl.quantize_delayed(xd[:r], "e4m3", odl.Ring(16), 0, 448.0, 1.0)
    r, dt, rate, _ = _grow(delayed, lambda r: r * cols * 3 + 80, 256, 8192, target_s / 2)
    out["legs"]["delayed_fp8_e4m3_transposed"] = {"GB/s": round(rate, 6), "cores": 1,
                                                  "sample": f"first {r} of 8192 rows, {dt:.2f} s"}
    del xd
    # Hadamard + MXFP4 column-wise: blocks run along the 8192 tokens, so samples are column strips
    g_bits, _, mask = workloads.weight_grad_operands()
    gx = workloads.bf16_to_f32(g_bits)

    def had(c):
        omx.quantize_colwise_t(gx[:, :c], "e2m1", "ceil", hadamard_mask=mask)
    c, dt, rate, _ = _grow(had, lambda c: 8192 * c * 2 + 8192 * c // 2 + 8192 * c // 32, 128, 4096, target_s / 2)
    out["legs"]["hadamard_mxfp4_colwise_one_operand"] = {"GB/s": round(rate, 6), "cores": 1,
                                                        "sample": f"first {c} of 4096 columns (all 8192 tokens), "
                                                                  f"{dt:.2f} s"}
    del gx
    # float64 GEMM reference (dequantized operands, BLAS) on leading rows of the MXFP8 MLP product
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:
        threadpool_limits = None
    threads = min(16, os.cpu_count() or 1)
    a_bits, w_bits = workloads.mlp_operands()
    qa, sa = omx.quantize_rowwise(workloads.bf16_to_f32(a_bits[:512]), "e4m3", "ceil")
    qw, sw = omx.quantize_rowwise(workloads.bf16_to_f32(w_bits), "e4m3", "ceil")
    del a_bits, w_bits

    def gemm(m):
        og.gemm_ref(qa[:m], sa[:m], "e4m3", qw, sw, "e4m3")
    if threadpool_limits is not None:
        with threadpool_limits(limits=threads):
            m, dt, _, _ = _grow(gemm, lambda m: 0, 64, 512, target_s / 2)
    else:
        m, dt, _, _ = _grow(gemm, lambda m: 0, 64, 512, target_s / 2)
        threads = None
    out["legs"]["gemm_fp64_reference_mxfp8_mlp"] = {
        "TFLOP/s": round(2.0 * m * 14336 * 4096 / dt / 1e12, 6), "threads": threads,
        "sample": f"first {m} of 8192 output rows of the 8192x14336x4096 product (float64 BLAS on the "
                  f"dequantized operands, dequantization included), {dt:.2f} s"}
    return out


if __name__ == "__main__":
    main()
