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
* Warm-up: exactly W untimed steps first (default 10000), then an untimed clock-settle phase
  of graph replays for at least 200 ms of wall time before every timed region, reported as
  "clock_settle". A step lasts microseconds, and the GPU's clocks need about a tenth of a
  second under load to rise: with a few warm-up steps alone the clocks were found at their
  low level (sclk 1096 MHz) and the same run was 9% slower.
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

from weight_only_quantized_dequant_amd import decode, inputs, wq  # noqa: E402

PEAK_HBM_GBS = 8000.0
METRIC = "weight-stream HBM GB/s (% of peak) for W8/W6/W4-A16 linear, M=1..16"
FMT_OF = {"w8": wq.FMT_W8, "w4g32": wq.FMT_W4G32, "w6e3m2": wq.FMT_W6E3M2, "w4e2m1": wq.FMT_W4E2M1,
          "w5e2m2": wq.FMT_W5E2M2, "f16": wq.FMT_F16}
# the same weights with bfloat16 activations ("_bf16"), and plain bfloat16 weights as their baseline
FMT_OF.update({k + "_bf16": v | wq.ACT_BF16 for k, v in list(FMT_OF.items()) if k != "f16"})
# int3 and the 2+4 split FP6 layout (fp16 activations only)
FMT_OF.update({"w3g32": wq.FMT_W3G32, "w6e3m2_p24": wq.FMT_W6E3M2_P24})
FMT_OF["bf16"] = wq.FMT_BF16 | wq.ACT_BF16


def is_bf16(code):
    return bool(code & wq.ACT_BF16)


def group_scaled(code):
    """Formats with a scale and a zero point per group of 32 K (int4, int3)."""
    return (code & 0xFF) in (wq.FMT_W4G32, wq.FMT_W3G32)


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
                    help="untimed steps before each timed region (a clock-settle phase of >= 200 ms follows them)")
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
    ap.add_argument("--decode", choices=["llama2_7b"], default=None,
                    help="time whole captured decode steps (embedding, every layer's norms, linears, rotary "
                         "embedding, attention over the key/value cache, the output layer and the next token) of a "
                         "random-init model, in tokens/s")
    ap.add_argument("--weights", default="w4g32", help="weight format of --decode")
    ap.add_argument("--context", type=int, default=512, help="cached positions when --decode starts timing")
    ap.add_argument("--max-seq", type=int, default=2048, help="key/value cache length of --decode")
    ap.add_argument("--read-floors", action="store_true",
                    help="time only the plain-read probe (libwq_probe.so) at the byte counts of the linears and "
                         "groups measured here, and an empty launch: the floors the design notes compare against")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain device copy of 512 MiB (a known-size kernel for counter calibration)")
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="length of the untimed clock-settle phase before each timed region (0 under a counter profiler)")
    ap.add_argument("--main-only", action="store_true",
                    help="time only the workload's step (no per-linear and no other-launch-style timings)")
    ap.add_argument("--summarize-counters", nargs="+", metavar="CSV", default=None,
                    help="no GPU work: print the per-kernel means of rocprofv3 --pmc counter_collection.csv files "
                         "as a markdown table (optionally only kernels containing --kernel-filter)")
    ap.add_argument("--kernel-filter", default=None)
    ap.add_argument("--counter-stat", choices=["mean", "max"], default="mean",
                    help="--summarize-counters: the mean per dispatch, or the largest dispatch")
    return ap.parse_args()


def summarize_counters(paths, kfilter=None, stat="mean"):
    """Per kernel name: dispatches, resources (VGPRs, AGPRs, LDS, scratch, grid and workgroup size)
    and the mean (or, stat="max", the largest) value per dispatch of every counter in rocprofv3
    counter-collection CSV files. The largest picks one dispatch out of many of the same kernel: the
    512 MiB copy of --copy-calibration among the smaller copies that set up the rotated weights."""
    import csv
    from collections import defaultdict
    vals = defaultdict(lambda: defaultdict(list))
    res = {}
    for path in paths:
        with open(path, newline="") as f:
            for row in csv.DictReader(f):
                k = row.get("Kernel_Name", "?")
                if kfilter and kfilter not in k:
                    continue
                vals[k][row["Counter_Name"]].append(float(row["Counter_Value"]))
                res.setdefault(k, {c: row.get(c) for c in ("VGPR_Count", "Accum_VGPR_Count", "SGPR_Count",
                                                          "LDS_Block_Size", "Scratch_Size", "Grid_Size",
                                                          "Workgroup_Size")})
    counters = sorted({c for k in vals for c in vals[k]})
    print("| kernel | dispatches | VGPR | AGPR | SGPR | LDS B | scratch | grid | wg | " + " | ".join(counters) + " |")
    print("|---|---:|---:|---:|---:|---:|---:|---:|---:|" + "---:|" * len(counters))
    for k in sorted(vals):
        n = max(len(v) for v in vals[k].values())
        r = res[k]
        agg = (lambda v: max(v)) if stat == "max" else (lambda v: sum(v) / len(v))
        cells = ["%.1f" % agg(vals[k][c]) if vals[k].get(c) else "" for c in counters]
        print("| %s | %d | %s | %s | %s | %s | %s | %s | %s | %s |" % (
            k[:90], n, r["VGPR_Count"], r["Accum_VGPR_Count"], r["SGPR_Count"], r["LDS_Block_Size"],
            r["Scratch_Size"], r["Grid_Size"], r["Workgroup_Size"], " | ".join(cells)))


CSRC = os.path.join(ROOT, "weight_only_quantized_dequant_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")


# The sources that define the decode-sized linear kernels (GEMV, fragment-load and LDS-staged
# matrix-core kernels) and the decoders they share; the prefill and decode-step kernels live in
# files of their own and do not change these kernels.
LINEAR_KERNEL_SOURCES = ("wq_device.h", "wq_internal.h", "wq_kernels.hip")


def kernel_source_hash():
    """sha256[:16] over the linear-kernel sources (LINEAR_KERNEL_SOURCES, in that order)."""
    import hashlib
    h = hashlib.sha256()
    for name in LINEAR_KERNEL_SOURCES:
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
    return decode.pack_host(fmt, w)


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


SETTLE_MS = [200.0]  # untimed load before every timed region, so that the GPU clocks have settled (--settle-ms)
SETTLE_LOG = []      # (ms, steps) of each settle phase, reported in the line


def time_steps(torch, run_step, steps, warmup, rot, spread=None):
    """Run `steps` steps as replays of graphs of `rot` steps; returns elapsed ms for exactly `steps` steps.
    Before the timed region: exactly `warmup` untimed steps, then an untimed clock-settle phase of
    replays until SETTLE_MS of wall time have passed (a step lasts microseconds; the GPU clocks need
    about a tenth of a second of load to rise, and a few warm-up steps alone left them low).
    With a list as `spread`, an event after every full replay also gives each replay's time per
    step in microseconds (appended to the list); the timed work is the same."""
    full = graph_of_steps(torch, run_step, 0, rot)
    rem = steps % rot
    tail = graph_of_steps(torch, run_step, 0, rem) if rem else None
    wfull, wrem = divmod(warmup, rot)
    for _ in range(wfull):
        full.replay()
    if wrem:
        graph_of_steps(torch, run_step, 0, wrem).replay()
    torch.cuda.synchronize()
    t0, settled = time.perf_counter(), 0
    while 1e3 * (time.perf_counter() - t0) < SETTLE_MS[0]:
        for _ in range(4):
            full.replay()
        settled += 4 * rot
        torch.cuda.synchronize()
    for _ in range(2):   # queued ahead of the timed region, so that the GPU does not idle before it
        full.replay()
    settled += 2 * rot
    SETTLE_LOG.append((1e3 * (time.perf_counter() - t0), settled))
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


def plain_read_floor(torch, nbytes, steps, warmup):
    """How fast a kernel that only reads does it for the same byte count: libwq_probe.so streams
    a buffer of nbytes with contiguous 1 KB wave loads, rotated over copies and timed exactly as
    the step is (graph replays, events). The fastest of a few wave counts and load depths is
    reported: the practical ceiling of a weight stream of this size on this GPU, against which
    the 8 TB/s peak alone overstates what any kernel of this size can reach."""
    import ctypes
    path = os.path.join(ROOT, "weight_only_quantized_dequant_amd", "libwq_probe.so")
    if not os.path.exists(path):
        raise RuntimeError("libwq_probe.so is missing: build with __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    lib.wq_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.wq_probe_read.restype = ctypes.c_int
    nb = nbytes // 16 * 16
    rot = max(1, math.ceil(ROTATE_BYTES / nb))
    bufs = [torch.full((nb,), i + 1, dtype=torch.uint8, device="cuda") for i in range(rot)]
    sink = torch.zeros(1 << 16, dtype=torch.int32, device="cuda")
    variants = {}
    for waves, unroll in ((4096, 2), (16384, 4), (32768, 2)):
        def run(i):
            st = lib.wq_probe_read(bufs[i % rot].data_ptr(), nb, waves, unroll, sink.data_ptr(), sink.numel(),
                                   ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
            if st != 0:
                raise RuntimeError("wq_probe_read failed: %d" % st)
        ms = time_steps(torch, run, steps, warmup, rot)
        variants["waves=%d,loads_in_flight=%d" % (waves, unroll)] = round(1e3 * ms / steps, 3)
    best = min(variants.values())
    del bufs, sink
    torch.cuda.empty_cache()
    return {"bytes": nb, "us": best, "GB/s": round(nb / best / 1e3, 1), "pct_of_peak": round(100 * nb / best / 1e3 / PEAK_HBM_GBS, 2),
            "us_by_variant": variants, "what": "the fastest plain read of the step's algorithmic bytes "
            "(libwq_probe.so, one contiguous span per wave), timed like the step"}


def run_read_floors(args, torch):
    """The plain-read floor (plain_read_floor) at the byte counts of single linears and grouped
    launches of both headline models, and the time per launch of a kernel that does nothing
    (1 and 1024 workgroups), all timed as the steps are (graph replays, events)."""
    import ctypes
    path = os.path.join(ROOT, "weight_only_quantized_dequant_amd", "libwq_probe.so")
    if not os.path.exists(path):
        raise RuntimeError("libwq_probe.so is missing: build with __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    lib.wq_probe_empty.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.wq_probe_empty.restype = ctypes.c_int
    sink = torch.zeros(16, dtype=torch.int32, device="cuda")
    steps = args.steps
    empty = {}
    for wg in (1, 1024):
        def run(i, wg=wg):
            st = lib.wq_probe_empty(wg, sink.data_ptr(), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
            if st != 0:
                raise RuntimeError("wq_probe_empty failed: %d" % st)
        # graphs of 100 launches: the launches run back to back, as the linears of a step do
        empty["workgroups=%d" % wg] = round(1e3 * time_steps(torch, run, steps, args.warmup, 100) / steps, 3)
    sizes = {}
    for name, fmt_name, shapes in (("llama7b_w4g32 4096x4096", "w4g32", [(4096, 4096)]),
                                   ("llama7b_w4g32 11008x4096", "w4g32", [(11008, 4096)]),
                                   ("llama7b_w4g32 group of 3", "w4g32", [(4096, 4096), (11008, 4096), (4096, 11008)]),
                                   ("llama7b_w8 group of 3", "w8", [(4096, 4096), (11008, 4096), (4096, 11008)]),
                                   ("llama70b_w6e3m2 group of 4", "w6e3m2", [(8192, 8192), (1024, 8192), (28672, 8192), (8192, 28672)])):
        fmt = FMT_OF[fmt_name]
        nbytes = sum(wq.wq_packed_bytes(fmt, n, k) + metadata_bytes(fmt, n, k) + 2 * k + 2 * n for n, k in shapes)
        f = plain_read_floor(torch, nbytes, steps, args.warmup)
        sizes[name] = {"bytes": f["bytes"], "us": f["us"], "GB/s": f["GB/s"], "pct_of_peak": f["pct_of_peak"]}
    print(json.dumps({"metric": "plain-read floor and empty-launch cost", "unit": "us", "steps": steps, "warmup": args.warmup,
                      "empty_launch_us": empty, "plain_read_floor": sizes,
                      "what": "libwq_probe.so kernels timed as graph replays with events on the launch stream; the floor "
                              "of a byte count is the fastest of three wave counts (bench.py plain_read_floor), the bytes "
                              "those of the linears' weights, metadata, x and y at M = 1",
                      "gpu": gpu_state(torch), "clock_settle": {"ms_min": round(min(t for t, _ in SETTLE_LOG), 1)}}))
    return 0


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


def host_cpu():
    """Cores this process may run on and the CPU model, as the host reports them."""
    cores = len(os.sched_getaffinity(0))
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return cores, model


def blas_on_host_cores():
    """Limit numpy's BLAS to the cores this process may use (its default may count more), so that
    the threads the oracle's product runs on are the host cores reported. Returns (context, threads)."""
    cores, _ = host_cpu()
    try:
        from threadpoolctl import threadpool_limits
        return threadpool_limits(limits=cores, user_api="blas"), cores
    except Exception:
        import contextlib
        return contextlib.nullcontext(), None


def cpu_baseline(code, linears_host, seconds):
    """The oracle (test infrastructure) timed on a bounded sample: per linear, a block of rows is
    unpacked, dequantized and multiplied in float64, repeated until `seconds` have passed."""
    import oracle  # the oracle is imported here only, for this reported baseline
    fmt = code & 0xFF
    act = oracle.ACT_BF16 if is_bf16(code) else oracle.ACT_F16
    dequant = oracle.dequant_bf16 if is_bf16(code) else oracle.dequant_fp16
    cores, cpu_model = host_cpu()
    limit, blas_threads = blas_on_host_cores()
    rows = 256
    work = []
    for (p, s, z, n, k, x) in linears_host:
        rb = wq.wq_packed_bytes(fmt, n, k) // n
        g = k // 32
        sl_s = None if s is None else (s[:rows * g] if group_scaled(fmt) else s[:rows])
        sl_z = None if z is None else z[:rows * g]
        work.append((p[:rows * rb], sl_s, sl_z, rows, k, x, rows * rb + 2 * (0 if s is None else sl_s.size)
                     + 2 * (0 if z is None else sl_z.size)))
    done_bytes, t0, reps = 0, time.perf_counter(), 0
    with limit:
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
    out = {"value": done_bytes / dt / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
           "cpu_model": cpu_model, "blas_threads": blas_threads,
           "sample": "%d rows of each linear (unpack + dequant + float64 product), %d passes in %.1f s; "
                     "elementwise steps single-threaded, the product on the BLAS threads (%s) over the %d host "
                     "cores this process may use" % (rows, reps, dt, blas_threads, cores)}
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
    # model (inputs.SWEEP_MODELS): formats, Ms, and the headline format
    "llama2_7b": (["f16", "w8", "w4g32", "w6e3m2", "w4e2m1", "w5e2m2"], [1], "w4g32"),
    "llama70b_w6": (["w6e3m2", "f16"], [1, 2, 4, 8, 16], "w6e3m2"),
}
# the launches of one decode-step layer, in order: q/k/v grouped, o, gate/up grouped, down
STEP_LAUNCHES = [("q", "k", "v"), ("o",), ("gate", "up"), ("down",)]


def host_bits16(t):
    return t.detach().cpu().contiguous().numpy().view(np.uint16)


def run_sweep(args, torch):
    """A decode step's linears of a random-init model: per layer q/k/v in one grouped call, o,
    gate/up in one grouped call, down. Every layer has its own weight memory (device copies
    of one seeded draw per shape: time depends only on shapes and bytes) and its own outputs, so
    the step streams the whole model from HBM. Timed as replays of a graph that holds one step.
    Unless --no-cpu, the outputs of the first and the last layer are then checked against the
    oracle and the oracle is timed on those two layers (sweep_oracle_leg)."""
    shapes, layers, _ = inputs.SWEEP_MODELS[args.sweep]
    fmts, ms_list, head_fmt = SWEEPS[args.sweep]
    if args.m is not None:
        ms_list = [args.m]
    name = {"llama2_7b": "llama2_7b_decode_sweep", "llama70b_w6": "llama70b_w6e3m2_decode_sweep"}[args.sweep]
    mmax = max(ms_list)
    draws = inputs.sweep_draws(args.sweep, mmax)
    xs = {k: torch.from_numpy(x.view(np.int16).copy()).to("cuda") for k, x in inputs.sweep_x(draws).items()}
    results, outs, steps = {}, {}, max(1, args.steps // 100)
    warm = max(2, args.warmup // 100)
    dev = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a).view(np.uint8)).to("cuda")
    for fname in fmts:
        fmt = FMT_OF[fname]
        proto = {}
        for (n, k), (w, _) in draws.items():
            proto[(n, k)] = tuple(dev(a) for a in pack(fmt, w))
        # one copy of every linear of every layer, each with its own output rows
        model = [{nm: tuple(None if t is None else t.clone() for t in proto[(n, k)]) +
                  (n, k, torch.empty((mmax, n), dtype=torch.int16, device="cuda")) for nm, n, k in shapes}
                 for _ in range(layers)]
        del proto
        step_bytes = layers * sum(wq.wq_packed_bytes(fmt, n, k) + metadata_bytes(fmt, n, k) for _, n, k in shapes)
        for m in (ms_list if fname != "f16" else ms_list[:1]):
            def item(lin):
                p, sc, z, n, k, y = lin
                return (xs[k][:m], p, sc, z, y[:m], n, k)

            def step(_i):
                for L in model:
                    for names in STEP_LAUNCHES:
                        wq.wq_linear_grouped([item(L[nm]) for nm in names], m, fmt)
            ms_total = time_steps(torch, step, steps, warm, 1)
            t = ms_total / steps
            results["%s_m%d" % (fname, m)] = {"ms_per_step": round(t, 4), "GB/s": round(step_bytes / (t * 1e-3) / 1e9, 1),
                                             "pct_of_peak": round(100 * step_bytes / (t * 1e-3) / 1e9 / PEAK_HBM_GBS, 2),
                                             "tok_per_s": round(m / (t * 1e-3), 1), "weight_GB": round(step_bytes / 1e9, 3),
                                             "launches_per_step": len(STEP_LAUNCHES) * layers}
            torch.cuda.synchronize()
            outs[(fname, m)] = {li: {nm: host_bits16(model[li][nm][5][:m]) for nm, _, _ in shapes}
                                for li in (0, layers - 1)}
        del model
        torch.cuda.empty_cache()
    for key, r in results.items():
        f16 = results.get("f16_m" + key.split("_m")[1])
        if f16 and not key.startswith("f16"):
            r["speedup_vs_f16"] = round(f16["ms_per_step"] / r["ms_per_step"], 3)
    head = "%s_m%d" % (head_fmt, ms_list[0])
    h = results[head]
    cpu, check = (None, None) if args.no_cpu else sweep_oracle_leg(args.sweep, draws, outs, head_fmt, ms_list[0])
    out = {"metric": METRIC, "value": h["GB/s"], "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": warm,
           "ms_per_step": h["ms_per_step"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "f16", "data": "synthetic", "pct_of_peak": h["pct_of_peak"],
           "config": {"workload": name, "weights": head_fmt, "M": ms_list[0], "layers": layers,
                      "linears_per_layer": [nm for nm, _, _ in shapes],
                      "launch": "per layer: grouped q/k/v, o, grouped gate/up, down",
                      "timing": "HIP graph of one decode step's linears, replayed; events on the launch stream"},
           "roofline": {"bound": "hbm", "achieved": h["GB/s"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": round(h["GB/s"] / PEAK_HBM_GBS, 4), "traffic": None, "kernel": "decode step (mixed)",
                        "launches_per_step": h["launches_per_step"]},
           "cpu_baseline": cpu, "oracle_check": check, "sweep": results,
           "clock_settle": {"ms_min": round(min(t for t, _ in SETTLE_LOG), 1), "timed_regions": len(SETTLE_LOG)}}
    print(json.dumps(out))
    return 0 if check is None or check["ok"] else 1


def sweep_oracle_leg(model, draws, outs, head_fmt, head_m):
    """The oracle beside a decode sweep (test infrastructure, imported here only).

    Check: for every format and M, the outputs of the first and the last layer on 64 sampled rows
    of each linear (plus its first and last row) against the oracle's own quantization of those
    rows of the fp32 draw (dequant, float64 product, closed-form bound and rtol = atol = 1e-2).
    cpu_baseline: the oracle as it stands (unpack + dequant + float64 product of every row of every
    linear, from the library's packed bytes) timed on the first and the last layer of the headline
    format and M; its results are compared with those two layers in full, and the time of a whole
    step is extrapolated from the two layers (labelled so)."""
    import oracle
    shapes, layers, _ = inputs.SWEEP_MODELS[model]
    xk = inputs.sweep_x(draws)
    check = {"layers": [0, layers - 1], "rows_per_linear": 66, "ok": True, "worst_err_over_bound": 0.0,
             "worst_err_over_tol": 0.0, "cases": 0}
    for (fname, m), per_layer in sorted(outs.items()):
        fmt = FMT_OF[fname] & 0xFF
        for li_shape, (nm, n, k) in enumerate(shapes):
            w, _ = draws[(n, k)]
            rows = np.unique(np.concatenate([[0, n - 1], np.random.default_rng([7, li_shape]).choice(n, 64, replace=False)]))
            _, s, z, codes = oracle.quantize_and_pack(fmt, w[rows])
            wd = oracle.dequant_fp16(fmt, codes, s, z)
            x = xk[k][:m]
            yref = oracle.linear_ref(x, wd)
            bound = oracle.error_bound(x, wd, yref)
            for li, ys in per_layer.items():
                err = np.abs(oracle.fp16_from_bits(ys[nm][:, rows]) - yref)
                rb = float((err / bound).max())
                rt = float((err / (1e-2 + 1e-2 * np.abs(yref))).max())
                check["worst_err_over_bound"] = max(check["worst_err_over_bound"], rb)
                check["worst_err_over_tol"] = max(check["worst_err_over_tol"], rt)
                check["cases"] += 1
                if not (rb <= 1.0 and rt <= 1.0 and np.all(np.isfinite(err))):
                    check["ok"] = False
                    check.setdefault("failed", []).append("%s m%d layer %d %s" % (fname, m, li, nm))
    # the headline format and M: the oracle on every row of the first and the last layer, timed
    fmt = FMT_OF[head_fmt] & 0xFF
    cores, cpu_model = host_cpu()
    limit, blas_threads = blas_on_host_cores()
    packs = {(n, k): pack(fmt, draws[(n, k)][0]) for (n, k) in draws}
    elapsed, wbytes, full_ok, worst = 0.0, 0, True, 0.0
    block = 2048
    with limit:
        for li in (0, layers - 1):
            ys = outs[(head_fmt, head_m)][li]
            for nm, n, k in shapes:
                p, s, z = packs[(n, k)]
                rb_bytes, g = wq.wq_packed_bytes(fmt, n, k) // n, k // 32
                x = xk[k][:head_m]
                for r0 in range(0, n, block):
                    r1 = min(n, r0 + block)
                    ss = None if s is None else (s[r0 * g:r1 * g] if group_scaled(fmt) else s[r0:r1])
                    zz = None if z is None else z[r0 * g:r1 * g]
                    t0 = time.perf_counter()
                    codes = oracle.unpack_vectorized(fmt, p[r0 * rb_bytes:r1 * rb_bytes], r1 - r0, k)
                    wd = oracle.dequant_fp16(fmt, codes, ss, zz)
                    yref = oracle.linear_ref(x, wd)
                    elapsed += time.perf_counter() - t0
                    bound = oracle.error_bound(x, wd, yref)
                    err = np.abs(oracle.fp16_from_bits(ys[nm][:, r0:r1]) - yref)
                    worst = max(worst, float((err / bound).max()))
                    full_ok &= bool(np.all(err <= bound))
                wbytes += wq.wq_packed_bytes(fmt, n, k) + metadata_bytes(fmt, n, k)
    check["full_layers"] = {"format": head_fmt, "M": head_m, "ok": full_ok, "worst_err_over_bound": worst}
    check["ok"] &= full_ok
    step_s = elapsed * layers / 2
    cpu = {"value": wbytes / elapsed / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle", "cpu_model": cpu_model,
           "blas_threads": blas_threads,
           "ms_per_step_extrapolated": round(1e3 * step_s, 1), "tok_per_s_extrapolated": head_m / step_s,
           "sample": "layers 0 and %d in full (%s, M=%d: unpack + dequant + float64 product of all %d linears, "
                     "%.1f s); the time of a %d-layer decode step is extrapolated x%d from these two layers"
                     % (layers - 1, head_fmt, head_m, len(shapes), elapsed, layers, layers // 2)}
    return cpu, check


def run_decode(args, torch):
    """Whole decode steps of a random-init model (weights of every layer in their own memory), one
    step captured as a HIP graph and replayed; each replay generates the next token of M sequences."""
    from weight_only_quantized_dequant_amd import decode
    cfg = dict(decode.LLAMA2_7B)
    fmt = FMT_OF[args.weights]
    m = args.m or 1
    S = args.max_seq
    steps = max(1, args.steps // 100)
    warm = max(1, min(args.warmup // 100, 100))
    host, _ = decode.random_model(cfg, fmt, 20, distinct_layers=1)
    dec = decode.Decoder(torch, cfg, fmt, m, S, *host)
    dec.tokens.fill_(1)
    graph = dec.capture()
    dec.pos.fill_(args.context)
    for _ in range(warm):
        graph.replay()
    torch.cuda.synchronize()
    t0, settled = time.perf_counter(), 0
    while 1e3 * (time.perf_counter() - t0) < SETTLE_MS[0] and args.context + settled + 1 < S - steps:
        graph.replay()
        settled += 1
        if settled % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    SETTLE_LOG.append((1e3 * (time.perf_counter() - t0), settled))
    dec.pos.fill_(args.context)       # the timed steps run at positions context .. context + steps - 1
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    logits = dec.logits.view(torch.float16).float()
    finite = bool(torch.isfinite(logits).all().item())
    wbytes = dec.weight_bytes()
    kv_bytes = 2 * cfg["layers"] * m * (args.context + steps // 2) * cfg["n_kv_heads"] * cfg["hd"] * 2
    out = {"metric": "decode tokens/s, whole captured decode step (Llama-2-7B shapes, random-init)",
           "value": round(m / (ms * 1e-3), 1), "unit": "tok/s", "n_gpus": 1, "steps": steps, "warmup": warm,
           "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "f16", "data": "synthetic",
           "config": {"workload": "llama2_7b_decode_step", "weights": args.weights, "M": m, "context": args.context,
                      "max_seq": S, "layers": cfg["layers"], "vocab": cfg["vocab"],
                      "launches_per_step": dec.launches_per_step(),
                      "timing": "HIP graph of one decode step, replayed; events on the launch stream"},
           "weight_GB_per_step": round(wbytes / 1e9, 3), "kv_cache_GB_read_per_step": round(kv_bytes / 1e9, 3),
           "weight_GB/s": round(wbytes / (ms * 1e-3) / 1e9, 1),
           "pct_of_peak_weights_and_cache": round(100 * (wbytes + kv_bytes) / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 2),
           "logits_finite": finite,
           "clock_settle": {"ms": round(SETTLE_LOG[-1][0], 1), "steps": SETTLE_LOG[-1][1]}}
    if not args.no_cpu:
        out["cpu_baseline"] = decode_cpu_baseline(cfg, fmt, host, args.context)
    print(json.dumps(out))
    return 0 if finite else 1


def decode_cpu_baseline(cfg, fmt, host, context):
    """The oracle (test infrastructure, imported here only) on one layer of the same model: unpack +
    dequant + float64 products of its seven linears, the norms, rotary embedding and attention over
    `context` cached positions, and the output layer; a whole step extrapolated from that layer."""
    import oracle
    from oracle import decode as D
    from weight_only_quantized_dequant_amd import decode
    cores, cpu_model = host_cpu()
    limit, blas_threads = blas_on_host_cores()
    layers, final_norm, lm_head, embed = host
    f = fmt & 0xFF
    L = layers[0]
    rng = np.random.default_rng(3)
    hd, H, Hkv, d = cfg["hd"], cfg["n_heads"], cfg["n_kv_heads"], cfg["d"]
    ck = D.f16(rng.standard_normal((1, context + 1, Hkv * hd)))
    cv = D.f16(rng.standard_normal((1, context + 1, Hkv * hd)))
    x = D.f16(rng.standard_normal((1, d)))

    def dq(pk, n, k):
        p, s, z = pk
        return oracle.dequant_fp16(f, oracle.unpack_vectorized(f, p, n, k), s, z)
    with limit:
        t0 = time.perf_counter()
        shapes = decode.device_shapes(cfg)
        W = {nm: dq(L[nm], *shapes[nm]) for nm in shapes}
        W["gate"], W["up"] = W["gu"][0::2], W["gu"][1::2]   # gate/up are held as interleaved rows
        h = D.rmsnorm(x, oracle.fp16_from_bits(L["attn_norm"]), cfg["eps"])
        q, k, v = D.lin(h, W["q"]), D.lin(h, W["k"]), D.lin(h, W["v"])
        ck[:, context] = D.f16(D.rope(k, context, hd, cfg["theta"]))
        cv[:, context] = v
        a = D.f16(D.attention(D.rope(q, context, hd, cfg["theta"]), ck, cv, context, H, Hkv, hd))
        x = x + D.lin(a, W["o"])
        h2 = D.rmsnorm(x, oracle.fp16_from_bits(L["ffn_norm"]), cfg["eps"])
        x = x + D.lin(D.silu_mul(D.lin(h2, W["gate"]), D.lin(h2, W["up"])), W["down"])
        t_layer = time.perf_counter() - t0
        t1 = time.perf_counter()
        D.lin(D.rmsnorm(x, oracle.fp16_from_bits(final_norm), cfg["eps"]), dq(lm_head, cfg["vocab"], d))
        t_out = time.perf_counter() - t1
    step_s = t_layer * cfg["layers"] + t_out
    return {"value": 1.0 / step_s, "unit": "tok/s", "cores": cores, "kind": "oracle", "cpu_model": cpu_model,
            "blas_threads": blas_threads, "extrapolated": True,
            "sample": "one decode layer (unpack + dequant + float64 products of its 7 linears, norms, rotary "
                      "embedding, attention over %d positions) in %.2f s and the output layer in %.2f s; a "
                      "%d-layer step extrapolated: %.1f s" % (context, t_layer, t_out, cfg["layers"], step_s)}


def main():
    args = parse()
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.kernel_filter, args.counter_stat)
        return 0
    if args.gpus != 1:
        print("bench.py measures one GPU only: libwq runs the linear on a single MI355X "
              "(no collectives); --gpus %d is not supported" % args.gpus, file=sys.stderr)
        return 2
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        return 1
    wq.lib()
    SETTLE_MS[0] = args.settle_ms
    if args.decode:
        return run_decode(args, torch)
    if args.sweep:
        return run_sweep(args, torch)
    if args.read_floors:
        return run_read_floors(args, torch)
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
    if not args.main_only:
        floor = plain_read_floor(torch, step_bytes, steps, args.warmup)
        floor["kernel_frac_of_floor"] = round(floor["us"] / (1e3 * avg_launch_ms * launches), 4)
        extras["plain_read_floor"] = floor
    # each linear alone (one launch per step, its own graph): per-shape durations and rates
    per_shape = {}
    for l in ([] if args.main_only else lins):
        ms_l = time_steps(torch, separate_step([l], rot), steps, args.warmup, rot)
        per_shape["%dx%d" % (l.n, l.k)] = {"us": round(1e3 * ms_l / steps, 3),
                                           "GB/s": round(l.weight_bytes * steps / (ms_l * 1e-3) / 1e9, 1)}
    extras["per_linear"] = per_shape
    if not args.main_only:
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
    out["clock_settle"] = {"ms_min": round(min(t for t, _ in SETTLE_LOG), 1), "timed_regions": len(SETTLE_LOG),
                           "steps_first_region": SETTLE_LOG[0][1],
                           "what": "untimed graph replays for >= %d ms of wall time after the warm-up steps, "
                                   "before every timed region" % SETTLE_MS[0]}
    out["gpu"] = state
    out.update(extras)
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
