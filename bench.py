#!/usr/bin/env python3
"""Benchmark of the weight-only-quantized linear (libwq) on one MI355X.

Metric: weight-stream HBM GB/s (and % of the 8 TB/s peak) of the fused dequant + linear.
A step is one pass of the device hot path over one batch. By default the batch is the
three Llama-7B-shaped W4 (int4, group 32) linears at M = 1 ([4096x4096], [11008x4096],
[4096x11008]). Quantize + pack happen once, offline, before
timing (the pages re-pack weights before inference).

Method:
* Weights are packed on the host by libwq and copied to HBM R times, with R * (bytes per
  step) >= 1 GiB. Step s reads copy s % R, so the 256 MB Infinity Cache cannot serve the
  weights from an earlier step: every step streams from HBM, as a real decode does.
* A step launches all linears of the workload in one wq_linear_grouped call (or, with
  --separate, one wq_linear call each). The K timed steps run as replays of a HIP graph
  that holds R steps (no host gaps), bracketed by synchronize + events on the launch
  stream. The other launch style and each linear alone are timed the same way and
  reported beside it.
* Warm-up: W untimed steps first (default 10000, about 0.15 s). A step lasts microseconds,
  and the GPU's clocks need that long under load to settle: with a few dozen warm-up steps
  the same run varied by +-5%.
* Roofline: the step holds only the dominant kernel's launches, back to back, so its
  average launch duration is the timed-region time per step over its launches.
* fp16 baselines: libwq's own fp16 kernel (grouped and separate) and torch's F.linear
  (hipBLASLt) on the same shapes, timed the same way.
* cpu_baseline: the CPU oracle (unpack + dequant + float64 product) on a bounded sample
  of rows of the same linears, on this host's cores.
Prints one JSON line.
"""

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from weight_only_quantized_dequant_amd import inputs, wq  # noqa: E402

PEAK_HBM_GBS = 8000.0
METRIC = "weight-stream HBM GB/s (% of peak) for W8/W6/W4-A16 linear, M=1..16"
FMT_OF = {"w8": wq.FMT_W8, "w4g32": wq.FMT_W4G32, "w6e3m2": wq.FMT_W6E3M2, "w4e2m1": wq.FMT_W4E2M1,
          "w5e2m2": wq.FMT_W5E2M2, "f16": wq.FMT_F16}
# the same weights with bfloat16 activations ("_bf16"), and plain bfloat16 weights as their baseline
FMT_OF.update({k + "_bf16": v | wq.ACT_BF16 for k, v in list(FMT_OF.items()) if k != "f16"})
FMT_OF["bf16"] = wq.FMT_BF16 | wq.ACT_BF16


def is_bf16(code):
    return bool(code & wq.ACT_BF16)


def bf16_bits(a):
    """float array -> bfloat16 bit patterns (torch's float32 -> bfloat16 rounding, nearest even)."""
    import torch
    f = torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.float32)))
    return f.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
ROTATE_BYTES = 1 << 30


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=4000)
    ap.add_argument("--warmup", type=int, default=10000,
                    help="untimed steps first; steps are microseconds long, and the GPU clocks need ~0.1 s of load to settle")
    ap.add_argument("--workload", default="llama7b_w4g32_linears", choices=sorted(inputs.WORKLOADS))
    ap.add_argument("--m", type=int, default=None, help="rows of x (default: the workload's first M)")
    ap.add_argument("--separate", action="store_true",
                    help="time one wq_linear call per linear instead of one grouped call per step")
    ap.add_argument("--no-baselines", action="store_true", help="skip the fp16 baselines")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle timing")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--sweep", choices=["llama2_7b", "llama70b_w6"], default=None,
                    help="time a whole decode step's linears of a random-init model instead of --workload: "
                         "llama2_7b (32 layers, fp16/W8/W4/W6, M=1) or llama70b_w6 (80 layers, W6, M=1..16)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain device copy of 512 MiB (a known-size kernel for counter calibration)")
    return ap.parse_args()


CSRC = os.path.join(ROOT, "weight_only_quantized_dequant_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")


def kernel_source_hash():
    """sha256[:16] over the device sources (csrc/*.hip and csrc/*.h, by name)."""
    import hashlib
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".h")):
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` from the committed counter summary (FETCH_SIZE + WRITE_SIZE,
    scaled by the same counters on a plain copy of known size), or None when there is no summary
    for this kernel and workload or the kernel source changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    e = rec.get("entries", {}).get("%s|%s" % (workload, kernel))
    if not e or rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return e.get("hbm_bytes_per_launch")


def metadata_bytes(fmt, n, k):
    return wq.wq_scales_bytes(fmt, n, k) + wq.wq_zeros_bytes(fmt, n, k)


def pack(fmt, w):
    """Quantize + pack fp32 W with libwq's host packers: (packed, scales or None, zeros or None)."""
    fmt &= 0xFF
    if fmt == wq.FMT_BF16:
        return bf16_bits(w).view(np.uint8).reshape(-1), None, None
    if fmt == wq.FMT_W8:
        return wq.wq_pack_int8(w) + (None,)
    if fmt == wq.FMT_W4G32:
        return wq.wq_pack_int4(w)
    if fmt == wq.FMT_W6E3M2:
        return wq.wq_pack_fp6(w) + (None,)
    if fmt == wq.FMT_W4E2M1:
        return wq.wq_pack_fp4(w) + (None,)
    if fmt == wq.FMT_W5E2M2:
        return wq.wq_pack_fp5(w) + (None,)
    return w.astype(np.float16).view(np.uint8).reshape(-1), None, None


class Linear:
    """One linear: packed weights (R rotation copies on the device) and its x, y buffers."""

    def __init__(self, torch, fmt, w, x_bits, copies):
        self.fmt = fmt
        self.n, self.k = w.shape
        self.m = x_bits.shape[0]
        p, s, z = pack(fmt, w)
        dev = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a).view(np.uint8)).to("cuda")
        p0, s0, z0 = dev(p), dev(s), dev(z)
        self.copies = [(p0, s0, z0)] + [(p0.clone(), None if s0 is None else s0.clone(), None if z0 is None else z0.clone())
                                        for _ in range(copies - 1)]
        self.x = torch.from_numpy(x_bits.view(np.int16).copy()).to("cuda")
        self.y = torch.empty((self.m, self.n), dtype=torch.int16, device="cuda")
        self.weight_bytes = wq.wq_packed_bytes(fmt, self.n, self.k) + metadata_bytes(fmt, self.n, self.k)
        self.io_bytes = 2 * self.m * self.k + 2 * self.m * self.n
        self.kernel = wq.wq_linear_kernel_name(fmt, self.m, self.n, self.k)

    def launch(self, copy, stream=None):
        p, s, z = self.copies[copy]
        wq.wq_linear(self.x, p, s, z, self.y, self.m, self.n, self.k, self.fmt, stream)


def graph_of_steps(torch, run_step, first, count):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run_step(first)                     # warm the launch path before capture
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            for i in range(count):
                run_step(first + i)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    return g


def time_steps(torch, run_step, steps, warmup, rot, spread=None):
    """Run `steps` steps as replays of graphs of `rot` steps; returns elapsed ms for exactly `steps` steps.
    With a list as `spread`, an event after every full replay also gives each replay's time per
    step in microseconds (appended to the list); the timed work is the same."""
    full = graph_of_steps(torch, run_step, 0, rot)
    rem = steps % rot
    tail = graph_of_steps(torch, run_step, 0, rem) if rem else None
    for _ in range(max(1, math.ceil(warmup / rot))):
        full.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    marks = []
    e0.record()
    for _ in range(steps // rot):
        full.replay()
        if spread is not None:
            marks.append(torch.cuda.Event(enable_timing=True))
            marks[-1].record()
    if tail is not None:
        tail.replay()
    e1.record()
    torch.cuda.synchronize()
    prev = e0
    for ev in marks:
        spread.append(1e3 * prev.elapsed_time(ev) / rot)
        prev = ev
    return e0.elapsed_time(e1)


def gpu_state(torch):
    """The device and its current clock levels and power as the kernel driver's sysfs files show
    them (plain file reads, best effort: no helper program is started)."""
    import glob
    props = torch.cuda.get_device_properties(0)
    state = {"name": props.name, "arch": getattr(props, "gcnArchName", None), "cus": props.multi_processor_count}
    sysfs = {}
    for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
        try:
            for clk in ("pp_dpm_sclk", "pp_dpm_mclk", "pp_dpm_fclk"):
                path = os.path.join(dev, clk)
                if os.path.exists(path):
                    cur = [l.strip() for l in open(path).read().splitlines() if l.strip().endswith("*")]
                    sysfs[clk] = cur[0] if cur else None
            for pw in glob.glob(os.path.join(dev, "hwmon", "hwmon*", "power1_average")) + \
                    glob.glob(os.path.join(dev, "hwmon", "hwmon*", "power1_input")):
                sysfs[os.path.basename(pw) + "_W"] = round(int(open(pw).read().strip()) / 1e6, 1)
        except (OSError, ValueError):
            continue
        if sysfs:
            break
    state["sysfs"] = sysfs or "unavailable"
    return state


def cpu_baseline(code, linears_host, seconds):
    """The oracle (test infrastructure) timed on a bounded sample: per linear, a block of rows is
    unpacked, dequantized and multiplied in float64, repeated until `seconds` have passed."""
    import oracle  # the oracle is imported here only, for this reported baseline
    fmt = code & 0xFF
    act = oracle.ACT_BF16 if is_bf16(code) else oracle.ACT_F16
    dequant = oracle.dequant_bf16 if is_bf16(code) else oracle.dequant_fp16
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([t.get("num_threads", 1) for t in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    rows = 256
    work = []
    for (p, s, z, n, k, x) in linears_host:
        rb = wq.wq_packed_bytes(fmt, n, k) // n
        g = k // 32
        sl_s = None if s is None else (s[:rows] if fmt != wq.FMT_W4G32 else s[:rows * g])
        sl_z = None if z is None else z[:rows * g]
        work.append((p[:rows * rb], sl_s, sl_z, rows, k, x, rows * rb + 2 * (0 if s is None else sl_s.size)
                     + 2 * (0 if z is None else sl_z.size)))
    done_bytes, t0, reps = 0, time.perf_counter(), 0
    while True:
        for (pp, ss, zz, r, k, x, b) in work:
            codes = oracle.unpack_vectorized(fmt, pp, r, k)
            wd = dequant(fmt, codes, ss, zz)
            oracle.linear_ref(x, wd, act=act)
            done_bytes += b
        reps += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    out = {"value": done_bytes / dt / 1e9, "unit": "GB/s", "cores": int(blas_threads), "kind": "oracle",
           "sample": "%d rows of each linear (unpack + dequant + float64 product), %d passes in %.1f s; "
                     "elementwise steps single-threaded, the product on %d BLAS threads" % (rows, reps, dt, blas_threads)}
    try:  # the same sample with the product on one thread, for a quarter of the time
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            b1, t1, r1 = 0, time.perf_counter(), 0
            while time.perf_counter() - t1 < seconds / 4:
                for (pp, ss, zz, r, k, x, b) in work:
                    oracle.linear_ref(x, dequant(fmt, oracle.unpack_vectorized(fmt, pp, r, k), ss, zz), act=act)
                    b1 += b
                r1 += 1
            out["single_thread"] = {"value": b1 / (time.perf_counter() - t1) / 1e9, "unit": "GB/s", "passes": r1}
    except Exception as e:
        out["single_thread"] = "unavailable (%s)" % type(e).__name__
    return out


SWEEPS = {
    # name: (layer shapes, layers, formats, Ms)
    "llama2_7b": (inputs.LLAMA2_7B_LINEARS, 32, ["f16", "w8", "w4g32", "w6e3m2", "w4e2m1", "w5e2m2"], [1]),
    "llama70b_w6": (inputs.LLAMA_70B_LINEARS, 80, ["w6e3m2", "f16"], [1, 2, 4, 8, 16]),
}


def run_sweep(args, torch):
    """A decode step's linears of a random-init model: per layer q/k/v in one grouped call, o,
    gate/up in one grouped call, down. Every layer has its own weight memory (device copies
    of one seeded draw per shape: time depends only on shapes and bytes), so the step streams
    the whole model from HBM. Timed as replays of a graph that holds one step."""
    shapes, layers, fmts, ms_list = SWEEPS[args.sweep]
    if args.m is not None:
        ms_list = [args.m]
    name = {"llama2_7b": "llama2_7b_decode_sweep", "llama70b_w6": "llama70b_w6e3m2_decode_sweep"}[args.sweep]
    distinct = sorted({(n, k) for _, n, k in shapes})
    draws = {}
    for i, (n, k) in enumerate(distinct):
        draws[(n, k)] = inputs.weights_and_x(inputs.rng_for(10 + list(SWEEPS).index(args.sweep), i), n, k, max(ms_list))
    mmax = max(ms_list)
    xs = {k: torch.from_numpy(draws[next(s for s in distinct if s[1] == k)][1].view(np.int16).copy()).to("cuda")
          for k in {k for _, k in distinct}}
    ys = {n: torch.empty((mmax, n), dtype=torch.int16, device="cuda") for n in {n for n, _ in distinct}}
    results, steps = {}, max(1, args.steps // 100)
    for fname in fmts:
        fmt = FMT_OF[fname]
        proto = {}
        for (n, k), (w, _) in draws.items():
            p, sc, z = pack(fmt, w)
            dev = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a).view(np.uint8)).to("cuda")
            proto[(n, k)] = (dev(p), dev(sc), dev(z))
        # one copy of every linear of every layer
        model = [{nm: tuple(None if t is None else t.clone() for t in proto[(n, k)]) + (n, k) for nm, n, k in shapes}
                 for _ in range(layers)]
        del proto
        step_bytes = layers * sum(wq.wq_packed_bytes(fmt, n, k) + metadata_bytes(fmt, n, k) for _, n, k in shapes)
        for m in (ms_list if fname != "f16" else ms_list[:1]):
            def item(lin):
                p, sc, z, n, k = lin
                return (xs[k][:m], p, sc, z, ys[n][:m], n, k)

            def step(_i):
                for L in model:
                    wq.wq_linear_grouped([item(L["q"]), item(L["k"]), item(L["v"])], m, fmt)
                    wq.wq_linear_grouped([item(L["o"])], m, fmt)
                    wq.wq_linear_grouped([item(L["gate"]), item(L["up"])], m, fmt)
                    wq.wq_linear_grouped([item(L["down"])], m, fmt)
            ms_total = time_steps(torch, step, steps, max(2, args.warmup // 100), 1)
            t = ms_total / steps
            results["%s_m%d" % (fname, m)] = {"ms_per_step": round(t, 4), "GB/s": round(step_bytes / (t * 1e-3) / 1e9, 1),
                                             "pct_of_peak": round(100 * step_bytes / (t * 1e-3) / 1e9 / PEAK_HBM_GBS, 2),
                                             "tok_per_s": round(m / (t * 1e-3), 1), "weight_GB": round(step_bytes / 1e9, 3),
                                             "launches_per_step": 4 * layers}
        del model
        torch.cuda.empty_cache()
    for key, r in results.items():
        f16 = results.get("f16_m" + key.split("_m")[1])
        if f16 and not key.startswith("f16"):
            r["speedup_vs_f16"] = round(f16["ms_per_step"] / r["ms_per_step"], 3)
    head = "w4g32_m1" if args.sweep == "llama2_7b" else "w6e3m2_m%d" % ms_list[0]
    h = results[head]
    out = {"metric": METRIC, "value": h["GB/s"], "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": max(2, args.warmup // 100),
           "ms_per_step": h["ms_per_step"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "f16", "data": "synthetic", "pct_of_peak": h["pct_of_peak"],
           "config": {"workload": name, "weights": head.split("_m")[0], "M": int(head.split("_m")[1]), "layers": layers,
                      "linears_per_layer": [nm for nm, _, _ in shapes],
                      "launch": "per layer: grouped q/k/v, o, grouped gate/up, down",
                      "timing": "HIP graph of one decode step's linears, replayed; events on the launch stream"},
           "roofline": {"bound": "hbm", "achieved": h["GB/s"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": round(h["GB/s"] / PEAK_HBM_GBS, 4), "traffic": None, "kernel": "decode step (mixed)",
                        "launches_per_step": h["launches_per_step"]},
           "cpu_baseline": None, "sweep": results}
    print(json.dumps(out))
    return 0


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: libwq runs the linear on a single MI355X "
              "(no collectives); --gpus %d is not supported" % args.gpus, file=sys.stderr)
        return 2
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        return 1
    wq.lib()
    if args.sweep:
        return run_sweep(args, torch)
    if args.copy_calibration:
        src = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    fmt_name, shapes, ms = inputs.WORKLOADS[args.workload]
    fmt = FMT_OF[fmt_name]
    m = args.m if args.m is not None else ms[0]
    stream_id = inputs.WORKLOAD_STREAM[args.workload]

    host = []
    for li, (n, k) in enumerate(shapes):
        w, x = inputs.weights_and_x(inputs.rng_for(stream_id, li), n, k, max(ms + [m]))
        if is_bf16(fmt):   # the same draws, rounded to bfloat16
            x = bf16_bits(x.view(np.float16).astype(np.float32))
        host.append((w, x[:m]))
    step_weight_bytes = sum(wq.wq_packed_bytes(fmt, n, k) + metadata_bytes(fmt, n, k) for n, k in shapes)
    rot = max(1, math.ceil(ROTATE_BYTES / step_weight_bytes))
    lins = [Linear(torch, fmt, w, x, rot) for (w, x) in host]
    step_io = sum(l.io_bytes for l in lins)

    def grouped_step(group, rotation):
        """One step: every linear of the workload in one wq_linear_grouped launch."""
        def run(i):
            items = []
            for l in group:
                p, sc, z = l.copies[i % rotation]
                items.append((l.x, p, sc, z, l.y, l.n, l.k))
            wq.wq_linear_grouped(items, m, group[0].fmt)
        return run

    def separate_step(group, rotation):
        """One step: one wq_linear launch per linear."""
        def run(i):
            for l in group:
                l.launch(i % rotation)
        return run

    steps = args.steps
    grouped = not args.separate
    step_fn = grouped_step(lins, rot) if grouped else separate_step(lins, rot)
    per_replay = []
    ms_total = time_steps(torch, step_fn, steps, args.warmup, rot, per_replay)
    value = step_weight_bytes * steps / (ms_total * 1e-3) / 1e9
    state = gpu_state(torch)   # right after the timed region, while the clocks are still up

    # roofline of the dominant kernel, from the same timed region: the step holds only this
    # kernel's launches, back to back in the graph, so its average duration is the step time
    # divided by its launches per step
    launches = 1 if grouped else len(lins)
    if grouped:
        dom_name = wq.wq_linear_grouped_kernel_name(fmt, m, shapes)
    else:
        dom_name = lins[0].kernel if len({l.kernel for l in lins}) == 1 else "mixed"
    step_bytes = step_weight_bytes + step_io
    avg_launch_ms = ms_total / steps / launches
    achieved = step_bytes / launches / (avg_launch_ms * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4),
                "traffic": measured_traffic(dom_name, args.workload),
                "kernel": dom_name, "launches_per_step": launches,
                "avg_launch_us": round(1e3 * avg_launch_ms, 3),
                "algorithmic_bytes_per_launch": int(step_bytes / launches)}

    extras = {}
    # each linear alone (one launch per step, its own graph): per-shape durations and rates
    per_shape = {}
    for l in lins:
        ms_l = time_steps(torch, separate_step([l], rot), steps, args.warmup, rot)
        per_shape["%dx%d" % (l.n, l.k)] = {"us": round(1e3 * ms_l / steps, 3),
                                           "GB/s": round(l.weight_bytes * steps / (ms_l * 1e-3) / 1e9, 1)}
    extras["per_linear"] = per_shape
    other = separate_step(lins, rot) if grouped else grouped_step(lins, rot)
    ms_other = time_steps(torch, other, steps, args.warmup, rot)
    extras["separate_calls" if grouped else "grouped_call"] = {
        "GB/s": round(step_weight_bytes * steps / (ms_other * 1e-3) / 1e9, 1), "ms_per_step": round(ms_other / steps, 5)}

    if not args.no_baselines:
        f16_bytes = sum(2 * n * k for n, k in shapes)
        rot16 = max(1, math.ceil(ROTATE_BYTES / f16_bytes))
        base16 = wq.FMT_BF16 | wq.ACT_BF16 if is_bf16(fmt) else wq.FMT_F16   # 16-bit weights of the activation type
        f16 = [Linear(torch, base16, w, x, rot16) for (w, x) in host]
        ms16g = time_steps(torch, grouped_step(f16, rot16), steps, args.warmup, rot16)
        ms16s = time_steps(torch, separate_step(f16, rot16), steps, args.warmup, rot16)
        # torch F.linear (hipBLASLt) on the same fp16 weights, same rotation
        import torch.nn.functional as F
        tdt = torch.bfloat16 if is_bf16(fmt) else torch.float16
        tw = [[c[0].view(tdt).view(l.n, l.k) for c in l.copies] for l in f16]
        tx = [l.x.view(tdt) for l in f16]
        def vendor_step(i):
            for j in range(len(f16)):
                F.linear(tx[j], tw[j][i % rot16])
        msv = time_steps(torch, vendor_step, steps, args.warmup, rot16)
        gbs = lambda ms_: round(f16_bytes * steps / (ms_ * 1e-3) / 1e9, 1)
        best16_ms = min(ms16g, ms16s, msv)
        bytes_ratio = f16_bytes / step_weight_bytes
        speedup = best16_ms / ms_total
        extras["fp16_baseline"] = {
            "libwq_f16_grouped": {"GB/s": gbs(ms16g), "ms_per_step": round(ms16g / steps, 5)},
            "libwq_f16_separate": {"GB/s": gbs(ms16s), "ms_per_step": round(ms16s / steps, 5)},
            "torch_F_linear": {"GB/s": gbs(msv), "ms_per_step": round(msv / steps, 5)},
            "speedup_vs_fastest_fp16": round(speedup, 3), "bytes_ratio": round(bytes_ratio, 3),
            "speedup_over_0.8x_bytes_ratio": round(speedup / (0.8 * bytes_ratio), 3)}
        del f16, tw, tx
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu:
        lh = []
        for (w, x), l in zip(host, lins):
            p0, s0, z0 = l.copies[0]
            to_np = lambda t, dt: None if t is None else t.cpu().numpy().view(dt)
            lh.append((to_np(p0, np.uint8), to_np(s0, np.uint16), to_np(z0, np.uint16), l.n, l.k, x))
        cpu = cpu_baseline(fmt, lh, args.cpu_seconds)

    flops = sum(2 * m * n * k for n, k in shapes)
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "ms_per_step": round(ms_total / steps, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if is_bf16(fmt) else "f16", "data": "synthetic",
        "pct_of_peak": round(100 * value / PEAK_HBM_GBS, 2),
        "config": {"workload": args.workload, "weights": fmt_name, "M": m,
                   "shapes_NxK": ["%dx%d" % s for s in shapes], "weight_bytes_per_step": step_weight_bytes,
                   "io_bytes_per_step": step_io, "rotation_copies": rot,
                   "tflops": round(flops * steps / (ms_total * 1e-3) / 1e12, 3),
                   "launch": "one wq_linear_grouped call per step" if grouped else "one wq_linear call per linear",
                   "timing": "HIP graph replays of %d steps, events on the launch stream" % rot},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    if per_replay:
        q = np.percentile(per_replay, [10, 50, 90])
        out["step_us_spread"] = {"p10": round(float(q[0]), 3), "p50": round(float(q[1]), 3), "p90": round(float(q[2]), 3),
                                 "replays": len(per_replay), "steps_per_replay": rot}
    out["gpu"] = state
    out.update(extras)
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
