#!/usr/bin/env python
"""Benchmark: one Qwen2.5-7B-shaped decode step of batch-1 W4A16 GEMVs on one MI355X.

A step is the whole hot path over one token: 28 layers x (fused qkv 4608x3584,
o 3584x3584, fused gate+up 37888x3584, down 3584x18944) plus an int4 lm_head
152064x3584, all int4 g=128 with fp16 scales and 4-bit zero points, M=1:
113 launches, stream-ordered and replayed as one captured graph. Each GEMV
uses the split count the library recommends (w4a16_splitk_choose): down
3584x18944 runs as w4a16_gemv_splitk, the others as w4a16_gemv.
The 3.68 GB of packed weights are distinct per layer and resident in HBM
before timing starts, so every step streams them from HBM (they exceed the
256 MB last-level cache). Inputs are seeded synthetic data with the
workload's laws (synthetic.py).

Prints one JSON line:
  value      = algorithmic bytes of the step / step time, GB/s (whole job),
  roofline   = the dominant kernel (the gate+up GEMV launch) timed with HIP
               events over back-to-back launches,
  cpu_baseline = the fp64 oracle on the host cores over a bounded sample of
               the same step (also used to check sampled outputs),
  chain      = the same 113 GEMVs as one persistent launch
               (w4a16_chain_run), each fed by its producer's output: us per
               step beside the graph's, and (in the cpu_baseline leg) every
               one of its 113 outputs against the oracle's bound.

  python bench.py [--steps K] [--warmup W]
  python bench.py --trace-summary DIR   # summarize a rocprofv3 kernel trace
"""
import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import synthetic  # noqa: E402

HBM_PEAK_GBPS = 8000.0  # MI355X published HBM3E bandwidth
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 matrix peak (no sparsity)
GROUP = 128
# Sources that decide the GEMV kernel's code and launch shape: a counter
# summary taken on other sources is not used.
KERNEL_SOURCES = [os.path.join(ROOT, "int4_weight_only_w4a16_amd", "csrc", f)
                  for f in ("gemv_kernel.h", "w4a16_device.h", "w4a16_internal.h", "api.cpp")]
COUNTERS_FILE = os.path.join(ROOT, "profiles", "gemv_gate_up_7b_counters.txt")


def algorithmic_bytes(M, N, K):
    """Minimum bytes of one GEMV: packed 4-bit weights, fp16 scales, 4-bit
    zeros, fp16 x and fp16 y (no padding)."""
    G = K // GROUP
    return N * K // 2 + 2 * N * G + N * G // 2 + 2 * M * K + 2 * M * N


def step_shapes():
    shapes = []
    for layer in range(synthetic.QWEN7B_LAYERS):
        for name, N, K in synthetic.QWEN7B_LAYER:
            shapes.append((f"L{layer}.{name}", N, K))
    shapes.append(synthetic.QWEN7B_LM_HEAD)
    return shapes


def kernel_digest():
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic():
    """Per-launch HBM traffic of the dominant kernel from the committed
    rocprofv3 counter summary, if it was taken on the current kernel source."""
    if not os.path.exists(COUNTERS_FILE):
        return None
    vals = {}
    for line in open(COUNTERS_FILE):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != kernel_digest():
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class Step:
    """Device buffers and the captured graph of one decode step."""

    def __init__(self, seed, torch):
        import int4_weight_only_w4a16_amd as w
        self.w, self.torch = w, torch
        dev = torch.device("cuda:0")
        self.shapes = step_shapes()
        self.bufs = []
        for i, (name, N, K) in enumerate(self.shapes):
            wq, sc, zp = synthetic.device_packed_weights(N, K, seed, i, dev)
            x = synthetic.device_activations(1, K, seed, i, dev)
            y = torch.empty((1, N), dtype=torch.int16, device=dev)
            self.bufs.append((name, N, K, wq, sc, zp, x, y))
        torch.cuda.synchronize()
        self.bytes = sum(algorithmic_bytes(1, N, K) for _, N, K in self.shapes)
        self.splits = {(N, K): w.w4a16_splitk_choose(1, N, K) for _, N, K in self.shapes}
        ws_bytes = max(w.w4a16_splitk_workspace_bytes(1, N, s) for (N, K), s in self.splits.items())
        self.ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)  # zero once; calls leave it zero
        self.stream = torch.cuda.Stream()

    def launch_all(self, stream, only=None, swiglu=False, torch_act=False, a8=None):
        for i, (name, N, K, wq, sc, zp, x, y) in enumerate(self.bufs):
            if only is not None and not name.endswith(only):
                continue
            if a8 == "fused":
                # INT8 activations quantized inside the GEMV launch.
                self.w.w4a16_gemv_a8_fused(1, N, K, wq, sc, zp, x, y, stream=stream)
            elif a8 is not None:
                # INT8-activation variant: quantize x (a launch of its own,
                # skipped for a8 == "gemv"), then the integer-MFMA GEMV.
                xq, sx, xs = self.a8_bufs[i]
                if a8 != "gemv":
                    self.w.w4a16_act_quant_i8(1, K, x, xq, sx, xs, stream=stream)
                self.w.w4a16_gemv_a8(1, N, K, wq, sc, zp, xq, sx, xs, y, stream=stream)
            elif swiglu and name.endswith("gate_up_proj"):
                # The same packed bytes read as the 16-row gate/up interleave.
                self.w.w4a16_gemv_swiglu(1, N // 2, K, wq, sc, zp, x, self.y_act, stream=stream)
            else:
                splits = self.splits[(N, K)]
                if splits > 1:
                    self.w.w4a16_gemv_splitk(1, N, K, splits, wq, sc, zp, x, y, self.ws, stream=stream)
                else:
                    self.w.w4a16_gemv(1, N, K, wq, sc, zp, x, y, stream=stream)
                if torch_act and name.endswith("gate_up_proj"):
                    # Comparison only: the unfused activation as separate
                    # torch elementwise kernels (silu, then the product).
                    h = y.view(self.torch.float16).view(1, 2, N // 2)
                    self.torch.mul(self.torch.nn.functional.silu(h[:, 0]), h[:, 1], out=self.y_act_h)

    def capture(self, only=None, swiglu=False, torch_act=False, a8=None):
        torch = self.torch
        if (swiglu or torch_act) and not hasattr(self, "y_act"):
            _, N, _ = synthetic.QWEN7B_LAYER[2]
            self.y_act = torch.empty((1, N // 2), dtype=torch.int16, device="cuda:0")
            self.y_act_h = self.y_act.view(torch.float16)
        if a8 is not None and not hasattr(self, "a8_bufs"):
            dev = torch.device("cuda:0")
            self.a8_bufs = [(torch.empty((1, K), dtype=torch.int8, device=dev),
                             torch.empty((1, K // 128), dtype=torch.float32, device=dev),
                             torch.empty((1, K // 128), dtype=torch.int32, device=dev))
                            for _, _, K, *_ in self.bufs]
        self.stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(self.stream):
            # warm: first launches load code objects (and, for the INT8
            # variant, leave valid codes for a8 == "gemv")
            self.launch_all(self.stream, only, swiglu, torch_act, None if a8 is None else "both")
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=self.stream):
                self.launch_all(self.stream, only, swiglu, torch_act, a8)
        torch.cuda.synchronize()
        return g

    def time_graph(self, g, reps, warmup):
        torch = self.torch
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(self.stream):
            e0.record(self.stream)
            for _ in range(reps):
                g.replay()
            e1.record(self.stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3  # seconds

    def time_eager(self, reps):
        torch = self.torch
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(self.stream):
            e0.record(self.stream)
            for _ in range(reps):
                self.launch_all(self.stream)
            e1.record(self.stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3


class ChainStep:
    """The same 113 GEMVs as one persistent launch (w4a16_chain_run), each
    reading the previous GEMV's output as its input: qkv the previous layer's
    down projection (the first one the step's external x), o the qkv output
    (standing for attention), gate/up + SwiGLU the o output, down the SwiGLU
    output, lm_head the last down output. Inputs are rescaled by 2^-shift
    on the way (an exact power of two) to keep fp16 in range. The down
    projection runs unsplit (three rounds per wave), the fastest measured."""

    SHIFTS = {"qkv_proj": 10, "o_proj": 3, "gate_up_proj": 3, "down_proj": 0, "lm_head": 10}

    def __init__(self, step, torch):
        w = step.w
        self.w, self.torch = w, torch
        dev = torch.device("cuda:0")
        self.ops = []
        last_down = -1
        for i, (name, N, K, wq, sc, zp, x, _) in enumerate(step.bufs):
            kind, n_out, src = w.CHAIN_GEMV, N, i - 1
            if name == "lm_head":
                src = last_down
            elif name.endswith("qkv_proj"):
                src = last_down
            elif name.endswith("gate_up_proj"):
                kind, n_out = w.CHAIN_SWIGLU, N // 2
            short = name.split(".")[-1]
            shift = self.SHIFTS[short] if src >= 0 else 0
            y = torch.full((1, n_out), -1, dtype=torch.int16, device=dev)
            self.ops.append(dict(kind=kind, N=n_out, K=K, splits=1, x_src=src, x_shift=shift, wq=wq, scales=sc,
                                 zeros=zp, x=x if src < 0 else None, y=y))
            if short == "down_proj":
                last_down = i
        plan, ws_bytes = w.w4a16_chain_plan(1, self.ops)
        self.plan = torch.from_numpy(plan).to(dev)
        self.ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
        self.stream = torch.cuda.Stream()

    def run(self):
        self.w.w4a16_chain_run(1, self.plan, self.ws, stream=self.stream)

    def time(self, reps, warmup):
        torch = self.torch
        for _ in range(warmup):
            self.run()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(self.stream)
        for _ in range(reps):
            self.run()
        e1.record(self.stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    def error_word(self):
        off = self.w.CHAIN_ERROR_OFFSET
        return int(self.ws[off:off + 4].cpu().numpy().view(np.uint32)[0])

    def outputs(self):
        return [o["y"].cpu().numpy().view(np.uint16).copy() for o in self.ops]


def handoff_costs(torch, seed, n=64, reps=20):
    """Cost of one dependency: n tiny GEMVs (128 x 128, 8 row tiles, one
    group), each reading the previous one's output, as one chain launch and
    as n launches in one graph; us per GEMV of each (almost no bytes: the
    time is the handoff and the fixed cost of a GEMV)."""
    import int4_weight_only_w4a16_amd as w
    dev = torch.device("cuda:0")
    N = K = 128
    wq, sc, zp = synthetic.device_packed_weights(N, K, seed, 8000, dev)
    xs = [synthetic.device_activations(1, K, seed, 8000, dev)]
    ys = [torch.empty((1, N), dtype=torch.int16, device=dev) for _ in range(n)]
    ops = [dict(kind=w.CHAIN_GEMV, N=N, K=K, splits=1, x_src=i - 1, x_shift=4 if i else 0, wq=wq, scales=sc,
                zeros=zp, x=xs[0] if i == 0 else None, y=ys[i]) for i in range(n)]
    plan, ws_bytes = w.w4a16_chain_plan(1, ops)
    plan_d = torch.from_numpy(plan).to(dev)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.Stream()
    for _ in range(3):
        w.w4a16_chain_run(1, plan_d, ws, stream=stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        w.w4a16_chain_run(1, plan_d, ws, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    chain_us = e0.elapsed_time(e1) * 1e3 / reps
    off = w.CHAIN_ERROR_OFFSET
    err = int(ws[off:off + 4].cpu().numpy().view(np.uint32)[0])
    # the same n GEMVs, each its own launch, in one graph (inputs chained through y as fp16)
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        for i in range(n):
            w.w4a16_gemv(1, N, K, wq, sc, zp, xs[0] if i == 0 else ys[i - 1], ys[i], stream=stream)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(n):
                w.w4a16_gemv(1, N, K, wq, sc, zp, xs[0] if i == 0 else ys[i - 1], ys[i], stream=stream)
    torch.cuda.synchronize()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    e0.record(stream)
    with torch.cuda.stream(stream):
        for _ in range(reps):
            g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    graph_us = e0.elapsed_time(e1) * 1e3 / reps
    return {"gemvs": n, "shape": f"{N}x{K}", "chain_us_per_dependent_gemv": round(chain_us / n, 3),
            "graph_us_per_dependent_launch": round(graph_us / n, 3), "chain_error_word": err}


def check_chain(chain, ys):
    """Every output of the chain against the oracle's bound, each GEMV's
    input being its producer's GPU output (first K columns) times 2^-shift,
    rounded to fp16 on the host (the chain's own input rule)."""
    import oracle
    orc = oracle.get()
    worst = 0.0
    for i, o in enumerate(chain.ops):
        M, N, K = 1, o["N"], o["K"]
        if o["x_src"] < 0:
            x_h = o["x"].cpu().numpy().view(np.uint16)
        else:
            y = np.ascontiguousarray(ys[o["x_src"]][:, :K]).view(np.float16).astype(np.float32)
            x_h = (y * np.float32(2.0 ** -o["x_shift"])).astype(np.float16).view(np.uint16)
        host = [t.cpu().numpy() for t in (o["wq"], o["scales"], o["zeros"])]
        wq_h, sc_h, zp_h = host[0], host[1].view(np.uint8), host[2]
        if o["kind"] == chain.w.CHAIN_SWIGLU:
            # packed rows: per 16-row tile, 8 gate rows then the 8 up rows of the same outputs
            NT = (N + 7) // 8
            r2, a2 = orc.gemv_packed(M, 16 * NT, K, wq_h, sc_h, zp_h, x_h)
            half = lambda a, h: a.reshape(M, NT, 2, 8)[:, :, h, :].reshape(M, 8 * NT)[:, :N]
            ref, bound = oracle.swiglu_bound(half(r2, 0), half(a2, 0), half(r2, 1), half(a2, 1))
            _, r = oracle.swiglu_report(ys[i], ref, bound, orc)
        else:
            ref, absref = orc.gemv_packed(M, N, K, wq_h, sc_h, zp_h, x_h)
            _, r = oracle.bound_report(ys[i], ref, absref, orc)
        worst = max(worst, r)
    return worst, len(chain.ops)


def cpu_baseline(step, budget_s):
    """The fp64 oracle, as it stands, over whole GEMVs of the same step in
    step order (lm_head first, then layers 0, 1, ...) until about budget_s
    seconds of oracle time are spent. Also checks those GEMVs' GPU outputs
    (from the last replay) against the oracle bound."""
    import oracle
    orc = oracle.get()
    order = [step.bufs[-1]] + step.bufs[:-1]
    done_bytes, spent, worst, names = 0, 0.0, 0.0, []
    for name, N, K, wq, sc, zp, x, y in order:
        host = [t.cpu().numpy() for t in (wq, sc, zp, x, y)]
        wq_h, sc_h, zp_h = host[0], host[1].view(np.uint8), host[2]
        x_h, y_h = host[3].view(np.uint16), host[4].view(np.uint16)
        t0 = time.perf_counter()
        ref, absref = orc.gemv_packed(1, N, K, wq_h, sc_h, zp_h, x_h)
        spent += time.perf_counter() - t0
        done_bytes += algorithmic_bytes(1, N, K)
        names.append(name)
        ok, r = oracle.bound_report(y_h, ref, absref, orc)
        worst = max(worst, r)
        if spent >= budget_s:
            break
    return {
        "value": round(done_bytes / spent / 1e9, 4),
        "unit": "GB/s",
        "cores": orc.num_threads(),
        "kind": "oracle",
        "sample": f"{len(names)} of the step's 113 GEMVs, whole ({names[0]}, {names[1] if len(names) > 1 else ''}"
                  f"{', ...' if len(names) > 2 else ''}), {done_bytes / 1e9:.3f} GB of algorithmic bytes, "
                  f"{spent:.1f} s of oracle time",
        "us_per_step_extrapolated": round(spent / done_bytes * step.bytes * 1e6, 1),
        "host": host_cpu(),
    }, worst, len(names)


def host_cpu():
    """The host's CPU model and logical CPU count, as the oracle's context."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return f"{model}, {os.cpu_count()} logical CPUs"



def trace_summary(directory):
    """Per-shape kernel durations from a rocprofv3 --kernel-trace CSV: the
    gemv kernel launches grouped by grid size (one grid size per shape)."""
    paths = glob.glob(os.path.join(directory, "**", "*kernel_trace.csv"), recursive=True)
    if not paths:
        raise SystemExit(f"no *kernel_trace.csv under {directory}")
    import csv
    groups = {}
    for path in paths:
        with open(path) as f:
            for row in csv.DictReader(f):
                name = row.get("Kernel_Name", "")
                if "w4a16" not in name:
                    continue
                dur = (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) * 1e-3  # us
                key = (name.split("(")[0][-60:], row.get("Grid_Size_X", row.get("Grid_Size", "?")),
                       row.get("Workgroup_Size_X", row.get("Workgroup_Size", "?")), row.get("Grid_Size_Y", "1"))
                groups.setdefault(key, []).append(dur)
    print(f"{'kernel':60s} {'grid_x':>10s} {'wg_x':>5s} {'calls':>6s} {'avg_us':>9s} {'med_us':>9s} {'min_us':>9s}"
          f" {'grid_y':>7s} {'p90_us':>9s} {'p99_us':>9s}")
    for key, durs in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        d = np.array(durs)
        print(f"{key[0]:60s} {key[1]:>10s} {key[2]:>5s} {len(d):6d} {d.mean():9.2f} {np.median(d):9.2f} {d.min():9.2f}"
              f" {key[3]:>7s} {np.percentile(d, 90):9.2f} {np.percentile(d, 99):9.2f}")


# Shapes of the counter pass, each launched COUNTER_REPS times in this order
# (with the library's split choice), so that a counter run's w4a16
# dispatches, in dispatch order, come in groups of COUNTER_REPS per shape.
COUNTER_REPS = 3
COUNTER_SHAPES = (
    [("7B qkv 4608x3584", 1, 4608, 3584, "gemv"), ("7B o 3584x3584", 1, 3584, 3584, "gemv"),
     ("7B gate_up 37888x3584", 1, 37888, 3584, "gemv"), ("7B gate_up+SwiGLU 37888x3584", 1, 18944, 3584, "swiglu"),
     ("7B down 3584x18944", 1, 3584, 18944, "gemv"), ("7B lm_head 152064x3584", 1, 152064, 3584, "gemv")]
    + [(f"27B {name} M={M}", M, N, K, "gemv") for M in synthetic.VERIFY_M if M in (1, 5, 8)
       for name, N, K in synthetic.VERIFY27B])


def counter_pass(torch, seed):
    """Launches every COUNTER_SHAPES entry COUNTER_REPS times, synchronously,
    for a rocprofv3 counter run (program directly after --)."""
    import int4_weight_only_w4a16_amd as w
    dev = torch.device("cuda:0")
    for i, (label, M, N, K, kind) in enumerate(COUNTER_SHAPES):
        rows = 16 * ((N + 7) // 8) if kind == "swiglu" else N
        wq, sc, zp = synthetic.device_packed_weights(rows, K, seed, 7000 + i, dev)
        x = synthetic.device_activations(M, K, seed, 7000 + i, dev)
        y = torch.empty((M, N), dtype=torch.int16, device=dev)
        splits = w.w4a16_splitk_choose(M, N, K) if kind == "gemv" else 1
        ws = torch.zeros(w.w4a16_splitk_workspace_bytes(M, N, max(splits, 2)), dtype=torch.uint8, device=dev)
        for _ in range(COUNTER_REPS):
            if kind == "swiglu":
                w.w4a16_gemv_swiglu(M, N, K, wq, sc, zp, x, y)
            elif splits > 1:
                w.w4a16_gemv_splitk(M, N, K, splits, wq, sc, zp, x, y, ws)
            else:
                w.w4a16_gemv(M, N, K, wq, sc, zp, x, y)
            torch.cuda.synchronize()
        print(f"counter pass: {label} M={M} splits={splits} x{COUNTER_REPS}", flush=True)
        del wq, sc, zp, x, y, ws


def _counter_rows(directory):
    import csv
    paths = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    if not paths:
        raise SystemExit(f"no *counter_collection.csv under {directory}")
    per = {}
    for path in paths:
        with open(path) as f:
            for row in csv.DictReader(f):
                d = per.setdefault(int(row["Dispatch_Id"]), {"name": row["Kernel_Name"],
                                                              "grid": row.get("Grid_Size", "?"),
                                                              "wg": row.get("Workgroup_Size", "?")})
                d[row["Counter_Name"]] = d.get(row["Counter_Name"], 0.0) + float(row["Counter_Value"])
    return [per[k] for k in sorted(per)]


def counter_summary(dirs):
    """Per-shape counters of the counter pass, one rocprofv3 run per directory
    (each with its own counters; a directory whose dispatches include the
    plain copy kernel of --copy-calibration gives the FETCH_SIZE and
    WRITE_SIZE scale factors instead)."""
    merged = [dict(label=l, M=M, N=N, K=K, kind=k) for l, M, N, K, k in COUNTER_SHAPES]
    scale = {}
    for directory in dirs:
        rows = _counter_rows(directory)
        w4 = [r for r in rows if "w4a16" in r["name"]]
        if not w4:
            # the copy kernel reads and writes 512 MiB (the fill before it reads nothing)
            for key in ("FETCH_SIZE", "WRITE_SIZE"):
                vals = [r[key] for r in rows if key in r]
                if vals:
                    scale[key] = (512 << 20) / (max(vals) * 1024)
            continue
        if len(w4) != COUNTER_REPS * len(COUNTER_SHAPES):
            raise SystemExit(f"{directory}: {len(w4)} w4a16 dispatches, expected {COUNTER_REPS * len(COUNTER_SHAPES)}")
        for i, m in enumerate(merged):
            group = w4[i * COUNTER_REPS:(i + 1) * COUNTER_REPS]
            m["grid"], m["wg"], m["kernel"] = group[0]["grid"], group[0]["wg"], group[0]["name"].split("(")[0][-70:]
            for key in group[0]:
                if key not in ("name", "grid", "wg"):
                    m[key] = sum(g[key] for g in group) / len(group)
    print(f"# scale factors from the plain copy kernel: {json.dumps({k: round(v, 4) for k, v in scale.items()})}")
    cols = ["label", "grid", "wg", "alg_MB", "fetch/alg", "write_KB", "tcc_hit%", "VALUBusy%", "lds_conf%",
            "wait/wave_cyc", "valu/wave", "mfma/wave"]
    print(" | ".join(cols))
    for m in merged:
        M, N, K = m["M"], m["N"], m["K"]
        rows = 16 * ((N + 7) // 8) if m["kind"] == "swiglu" else N
        alg = algorithmic_bytes(M, rows, K) if m["kind"] != "swiglu" else algorithmic_bytes(M, rows, K) - 2 * M * rows + 2 * M * N
        out = [m["label"], str(m.get("grid", "?")), str(m.get("wg", "?")), f"{alg / 1e6:.2f}"]
        f = m.get("FETCH_SIZE")
        out.append(f"{f * 1024 * scale.get('FETCH_SIZE', 1.0) / alg:.4f}" if f is not None else "-")
        wr = m.get("WRITE_SIZE")
        out.append(f"{wr * scale.get('WRITE_SIZE', 1.0):.1f}" if wr is not None else "-")
        hit, miss = m.get("TCC_HIT_sum"), m.get("TCC_MISS_sum")
        out.append(f"{100 * hit / (hit + miss):.1f}" if hit is not None and miss is not None and hit + miss > 0 else "-")
        out.append(f"{m['VALUBusy']:.1f}" if "VALUBusy" in m else "-")
        bc, lds = m.get("SQ_LDS_BANK_CONFLICT"), m.get("SQ_ACTIVE_INST_LDS")
        out.append(f"{100 * bc / lds:.1f}" if bc is not None and lds else "-")
        wt, wc = m.get("SQ_WAIT_INST_ANY"), m.get("SQ_WAVE_CYCLES")
        out.append(f"{wt / wc:.3f}" if wt is not None and wc else "-")
        waves = m.get("SQ_WAVES")
        out.append(f"{m['SQ_INSTS_VALU'] / waves:.0f}" if waves and "SQ_INSTS_VALU" in m else "-")
        out.append(f"{m['SQ_INSTS_MFMA'] / waves:.0f}" if waves and "SQ_INSTS_MFMA" in m else "-")
        print(" | ".join(out))


def gemm_counter_summary(dirs, fetch_scale=1.9998, write_scale=1.0):
    """Per-dispatch counter means of the M = 2048 prefill GEMMs (128-row
    tiles) in rocprofv3 --pmc runs of `bench.py --prefill-gemm`, one run per
    directory, for gate+up 37888x3584 and down 3584x18944. FETCH_SIZE and
    WRITE_SIZE are scaled by the plain copy kernel's factors (the GEMV
    counter file's)."""
    M = 2048
    shapes = {"gate+up 37888x3584": (37888, 3584), "down 3584x18944": (3584, 18944)}
    grids = {name: str((M + 127) // 128 * 256 * ((N + 127) // 128)) for name, (N, K) in shapes.items()}
    vals = {name: {} for name in shapes}
    for directory in dirs:
        for r in _counter_rows(directory):
            if "gemm_kernel" not in r["name"]:
                continue
            for name, g in grids.items():
                if r["grid"] == g:
                    for k, v in r.items():
                        if k not in ("name", "grid", "wg"):
                            vals[name].setdefault(k, []).append(v)
    mean = {name: {k: sum(v) / len(v) for k, v in d.items()} for name, d in vals.items()}
    count = {name: {k: len(v) for k, v in d.items()} for name, d in vals.items()}
    names = list(shapes)
    print(f"{'':40s}" + "".join(f"{n:>24s}" for n in names))

    def row(label, f, fmt="{:,.0f}"):
        cells = []
        for n in names:
            try:
                cells.append(fmt.format(f(mean[n], *shapes[n])))
            except (KeyError, ZeroDivisionError):
                cells.append("-")
        print(f"{label:40s}" + "".join(f"{c:>24s}" for c in cells))

    disp = {n: min(count[n].values()) if count[n] else 0 for n in names}
    print(f"{'dispatches averaged':40s}" + "".join(f"{disp[n]:>24d}" for n in names))
    row("SQ_WAVES", lambda d, N, K: d["SQ_WAVES"])
    row("SQ_INSTS_MFMA", lambda d, N, K: d["SQ_INSTS_MFMA"])
    row("  M*N*K / (16*16*32)", lambda d, N, K: M * N * K / (16 * 16 * 32))
    row("SQ_INSTS_VALU (includes MFMA)", lambda d, N, K: d["SQ_INSTS_VALU"])
    row("  other VALU per MFMA", lambda d, N, K: (d["SQ_INSTS_VALU"] - d["SQ_INSTS_MFMA"]) / d["SQ_INSTS_MFMA"],
        "{:.2f}")
    row("SQ_INSTS_LDS", lambda d, N, K: d["SQ_INSTS_LDS"])
    row("SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE %",
        lambda d, N, K: 100 * d["SQ_LDS_BANK_CONFLICT"] / d["SQ_LDS_IDX_ACTIVE"], "{:.2f}")
    row("SQ_VALU_MFMA_BUSY_CYCLES", lambda d, N, K: d["SQ_VALU_MFMA_BUSY_CYCLES"])
    row("  / (1024 SIMDs x 2.4 GHz), us", lambda d, N, K: d["SQ_VALU_MFMA_BUSY_CYCLES"] / 1024 / 2.4e3, "{:.1f}")
    row("  flops / 2.5 PFLOP/s, us", lambda d, N, K: 2.0 * M * N * K / (MFMA_F16_PEAK_TFLOPS * 1e6), "{:.1f}")
    row("SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES %", lambda d, N, K: 100 * d["SQ_WAIT_INST_ANY"] / d["SQ_WAVE_CYCLES"],
        "{:.1f}")
    row("SQ_ACTIVE_INST_ANY / SQ_WAVE_CYCLES %",
        lambda d, N, K: 100 * d["SQ_ACTIVE_INST_ANY"] / d["SQ_WAVE_CYCLES"], "{:.1f}")
    row("SQ_INSTS_VMEM_RD per wave", lambda d, N, K: d["SQ_INSTS_VMEM_RD"] / d["SQ_WAVES"])
    row("FETCH_SIZE (KiB)", lambda d, N, K: d["FETCH_SIZE"])
    row("WRITE_SIZE (KiB)", lambda d, N, K: d["WRITE_SIZE"])
    row("  M*N*2 B / 1024", lambda d, N, K: M * N * 2 / 1024)
    row("scaled L2-miss reads (B)", lambda d, N, K: d["FETCH_SIZE"] * 1024 * fetch_scale)
    row("algorithmic reads: weights + x (B)", lambda d, N, K: algorithmic_bytes(M, N, K) - 2 * M * N)
    row("  reads / algorithmic reads", lambda d, N, K: d["FETCH_SIZE"] * 1024 * fetch_scale /
        (algorithmic_bytes(M, N, K) - 2 * M * N), "{:.2f}")


def read_ceiling_gbps(torch):
    """Plain-read ceiling of this device: the library's read probe (the
    GEMV's own non-temporal 16-byte loads, nothing stored) over 1 GiB at four
    grid sizes, the best of all; the kernels are compared with it beside the
    peak. (Two to three workgroups per CU read fastest, about 7.1 TB/s; from
    4 on it drops to about 6.)"""
    import int4_weight_only_w4a16_amd as w
    rbuf = torch.ones(1 << 30, dtype=torch.uint8, device="cuda:0")
    sink = torch.zeros(16, dtype=torch.uint8, device="cuda:0")
    best = 0.0
    for grid in (256, 512, 768, 1024):
        w.w4a16_read_probe(rbuf, grid, sink)
        torch.cuda.synchronize()
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(4):
                w.w4a16_read_probe(rbuf, grid, sink)
            e1.record()
            torch.cuda.synchronize()
            best = max(best, 4 * (1 << 30) / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del rbuf, sink
    return best


def decompose_pass(torch, seed, steps):
    """`steps` graph replays of the 7B step, then `steps` eager steps (the
    same 113 launches from the host), for a rocprofv3 --kernel-trace run;
    then both timed with HIP events without the profiler's help, and the
    plain-read ceiling, printed as one JSON line."""
    step = Step(seed, torch)
    graph = step.capture()
    torch.cuda.synchronize()
    for _ in range(steps):
        graph.replay()
    torch.cuda.synchronize()
    with torch.cuda.stream(step.stream):
        for _ in range(steps):
            step.launch_all(step.stream)
    torch.cuda.synchronize()
    g_s = step.time_graph(graph, 50, 5) / 50
    e_s = step.time_eager(50) / 50
    print(json.dumps({"graph_us_per_step": round(g_s * 1e6, 2), "eager_us_per_step": round(e_s * 1e6, 2),
                      "bytes_per_step": step.bytes, "read_ceiling_GBps": round(read_ceiling_gbps(torch), 1),
                      "launches_per_step": len(step.shapes), "steps_traced_each": steps}), flush=True)


def _graph_cold_us(torch, launch, n, rounds=5, reps=3):
    """Median microseconds per launch of `launch(stream)`, which makes `n`
    launches over distinct buffers (more bytes than the caches hold), captured
    once in a graph and replayed `reps` times per round."""
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        launch(stream)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            launch(stream)
        torch.cuda.synchronize()
        g.replay()
        g.replay()
        torch.cuda.synchronize()
        ts = []
        for _ in range(rounds):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3 / (reps * n))
    del g
    return sorted(ts)[len(ts) // 2]


def read_floor(torch, seed):
    """Per 7B-shaped GEMV of the decode step: the time a plain read of its
    weight, scale and zero bytes takes (the library's read probe at its best
    grid), against the GEMV itself, both as back-to-back launches over
    distinct cold buffers in one graph; the split-K GEMV of down at several
    split counts; and the step both add up to (28 layers and lm_head). One
    JSON line per shape, then one for the step."""
    import int4_weight_only_w4a16_amd as w
    dev = torch.device("cuda:0")
    sink = torch.zeros(16, dtype=torch.uint8, device=dev)
    shapes = [(name, N, K) for name, N, K in synthetic.QWEN7B_LAYER] + [synthetic.QWEN7B_LM_HEAD]
    sums = {"read": 0.0, "gemv": 0.0}
    for name, N, K in shapes:
        G = K // GROUP
        nb = N * K // 2 + 2 * N * G + N * G // 2
        copies = max(2, (768 << 20) // nb + 1)
        bufs = [torch.ones((nb + 4095) // 4096 * 4096, dtype=torch.uint8, device=dev) for _ in range(copies)]
        by_grid = {}
        for grid in (256, 512, 768, 1024, 2048, 4096):
            by_grid[grid] = _graph_cold_us(
                torch, lambda st, grid=grid: [w.w4a16_read_probe(b, grid, sink, nbytes=nb, stream=st) for b in bufs],
                copies)
        del bufs
        sets = [synthetic.device_packed_weights(N, K, seed, 700 + c, dev) for c in range(copies)]
        x = synthetic.device_activations(1, K, seed, 1, dev)
        y = torch.empty((1, N), dtype=torch.int16, device=dev)
        gemv = _graph_cold_us(torch, lambda st: [w.w4a16_gemv(1, N, K, *a, x, y, stream=st) for a in sets], copies)
        row = {"shape": f"{name} {N}x{K}", "bytes": nb, "copies": copies,
               "read_us_by_grid": {g: round(t, 2) for g, t in by_grid.items()},
               "read_us": round(min(by_grid.values()), 2), "gemv_us": round(gemv, 2),
               "gemv_over_read_us": round(gemv - min(by_grid.values()), 2)}
        if name == "down_proj":
            ws = torch.zeros(w.w4a16_splitk_workspace_bytes(1, N, 16), dtype=torch.uint8, device=dev)
            row["gemv_splitk_us"] = {s: round(_graph_cold_us(
                torch, lambda st, s=s: [w.w4a16_gemv_splitk(1, N, K, s, *a, x, y, ws, stream=st) for a in sets],
                copies), 2) for s in (2, 4, 8, 16)}
        print(json.dumps(row), flush=True)
        times = 1 if (name, N, K) == synthetic.QWEN7B_LM_HEAD else synthetic.QWEN7B_LAYERS
        sums["read"] += times * min(by_grid.values())
        sums["gemv"] += times * gemv
        del sets
    total = sum(algorithmic_bytes(1, N, K) for _, N, K in step_shapes())
    print(json.dumps({"step_launches": len(step_shapes()), "step_read_only_us": round(sums["read"], 1),
                      "step_gemv_us": round(sums["gemv"], 1), "step_bytes": total,
                      "step_at_80pct_of_peak_us": round(total / (0.8 * HBM_PEAK_GBPS) / 1e3, 1)}), flush=True)


def decompose_summary(directory, steps, launches=113):
    """Step decomposition from a kernel trace of decompose_pass: per step,
    the wall span, the sum of kernel durations and the gaps between
    consecutive kernels, for the graph steps and the eager steps."""
    import csv
    paths = glob.glob(os.path.join(directory, "**", "*kernel_trace.csv"), recursive=True)
    if not paths:
        raise SystemExit(f"no *kernel_trace.csv under {directory}")
    ev = []
    for path in paths:
        with open(path) as f:
            for row in csv.DictReader(f):
                if "w4a16" in row.get("Kernel_Name", ""):
                    ev.append((int(row["Start_Timestamp"]), int(row["End_Timestamp"])))
    ev.sort()
    # The capture's eager warm-up step comes first, then the traced graph and
    # eager steps; the timed runs (and the read probe) follow them.
    ev = ev[launches:launches + 2 * steps * launches]
    for label, part in (("graph", ev[:steps * launches]), ("eager", ev[steps * launches:])):
        spans, busy, gaps = [], [], []
        for s0 in range(0, len(part), launches):
            st = part[s0:s0 + launches]
            spans.append((st[-1][1] - st[0][0]) * 1e-3)
            busy.append(sum(e - b for b, e in st) * 1e-3)
            gaps.extend((st[i][0] - st[i - 1][1]) * 1e-3 for i in range(1, len(st)))
        g = np.array(gaps)
        print(f"{label}: steps {len(spans)}, span us median {np.median(spans):.1f}, kernel busy us median "
              f"{np.median(busy):.1f}, gaps per step us median {np.median(spans) - np.median(busy):.1f}; "
              f"gap between kernels us: median {np.median(g):.2f} p10 {np.percentile(g, 10):.2f} "
              f"p90 {np.percentile(g, 90):.2f} min {g.min():.2f}")


def oracle_set(one, M, budget_s):
    """The oracle over whole GEMVs of one set (in set order) until about
    budget_s seconds of oracle time: (seconds, algorithmic bytes, GEMVs,
    worst GPU error over the bound)."""
    import oracle
    orc = oracle.get()
    spent, done_bytes, n, worst = 0.0, 0, 0, 0.0
    for N, K, wq, sc, zp, x, y, _ in one:
        wq_h, sc_h, zp_h, x_h, y_h = (t.cpu().numpy() for t in (wq, sc, zp, x, y))
        t0 = time.perf_counter()
        ref, absref = orc.gemv_packed(M, N, K, wq_h, sc_h.view(np.uint8), zp_h, x_h.view(np.uint16))
        spent += time.perf_counter() - t0
        done_bytes += algorithmic_bytes(M, N, K)
        n += 1
        _, r = oracle.bound_report(y_h.view(np.uint16), ref, absref, orc)
        worst = max(worst, r)
        if spent >= budget_s:
            break
    return spent, done_bytes, n, worst, orc.num_threads()


def run_configs(torch, seed, oracle_budget_s=3.0):
    """Every workload configuration, warm and cold, µs and GB/s per set.

    A set is the configuration's GEMVs launched back to back on one stream,
    with the library's split choice. Warm: one copy of the weights, the set
    repeated in one captured graph of at least 64 launches (inputs stay in
    the 256 MB last-level cache where they fit). Cold: distinct weight copies
    totalling at least 1 GiB, each set once per graph replay, so every
    replay streams from HBM. Every graph is timed in 5 rounds (5 replays
    each), the measurements in a seeded random order within each round; a
    row reports the median and the mean of its rounds and flags a mean more
    than 15% away from the median. Each row also carries the fp64 oracle
    timed on the host cores over the set's GEMVs (whole GEMVs, up to about
    oracle_budget_s seconds, extrapolated to the set) and checks those
    GEMVs' GPU outputs against the oracle's bound.
    Configuration 4 (the whole 7B step) is the default bench line."""
    import int4_weight_only_w4a16_amd as w
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream()
    GiB = 1 << 30

    def build(shapes, M, copies, tid0):
        sets = []
        for c in range(copies):
            one = []
            for i, (name, N, K) in enumerate(shapes):
                wq, sc, zp = synthetic.device_packed_weights(N, K, seed, tid0 + 1000 * c + i, dev)
                x = synthetic.device_activations(M, K, seed, tid0 + i, dev)
                y = torch.empty((M, N), dtype=torch.int16, device=dev)
                one.append((N, K, wq, sc, zp, x, y, w.w4a16_splitk_choose(M, N, K)))
            sets.append(one)
        ws_bytes = max(w.w4a16_splitk_workspace_bytes(M, N, 2) for _, N, K in shapes)
        ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
        return sets, ws

    def launch(sets, ws, M, reps):
        for _ in range(reps):
            for one in sets:
                for N, K, wq, sc, zp, x, y, splits in one:
                    if splits > 1:
                        w.w4a16_gemv_splitk(M, N, K, splits, wq, sc, zp, x, y, ws, stream=stream)
                    else:
                        w.w4a16_gemv(M, N, K, wq, sc, zp, x, y, stream=stream)

    def capture(sets, ws, M, reps_in_graph):
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            launch(sets, ws, M, 1)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                launch(sets, ws, M, reps_in_graph)
        torch.cuda.synchronize()
        return g

    def time_graph(g, launches_per_replay_in_sets, replays):
        for _ in range(2):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e0.record(stream)
            for _ in range(replays):
                g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (replays * launches_per_replay_in_sets)  # µs per set

    configs = [
        ("1: single GEMV 896x896", [("single", 896, 896)], (1,)),
        ("2: Qwen2.5-0.5B decode linear set, 24 layers x 7", [
            (f"L{l}.{n}", N, K) for l in range(synthetic.QWEN05B_LAYERS) for n, N, K in synthetic.QWEN05B_LAYER], (1,)),
        ("2 (variant): the same with q/k/v and gate/up each packed as one matrix, 24 layers x 4", [
            (f"L{l}.{n}", N, K) for l in range(synthetic.QWEN05B_LAYERS)
            for n, N, K in (("qkv_proj", 896 + 2 * 128, 896), ("o_proj", 896, 896), ("gate_up_proj", 2 * 4864, 896),
                            ("down_proj", 896, 4864))], (1,)),
        ("3: Qwen2.5-7B layer (qkv, o, gate_up, down)", list(synthetic.QWEN7B_LAYER), (1,)),
        ("5: 27B-class verify pair (up 17408x5120, down 5120x17408)", list(synthetic.VERIFY27B), synthetic.VERIFY_M),
    ]
    import random
    rows, items = [], []  # items: (row index, "warm"/"cold", graph, sets per replay, kept buffers)
    for ci, (label, shapes, Ms) in enumerate(configs):
        for M in Ms:
            nbytes = sum(algorithmic_bytes(M, N, K) for _, N, K in shapes)
            launches = len(shapes)
            rows.append({"config": label, "M": M, "launches_per_set": launches, "bytes_per_set": nbytes})
            sets, ws = build(shapes, M, 1, 100 * ci)
            reps = -(-64 // launches)  # at least 64 launches per replay (a replay has a fixed cost)
            items.append((len(rows) - 1, "warm", capture(sets, ws, M, reps), reps, (sets, ws)))
            copies = -(-GiB // nbytes)
            rows[-1]["cold_copies"] = copies
            sets, ws = build(shapes, M, copies, 100 * ci)
            items.append((len(rows) - 1, "cold", capture(sets, ws, M, 1), copies, (sets, ws)))
    rng = random.Random(seed)
    times = {}
    for rnd in range(5):
        order = list(range(len(items)))
        rng.shuffle(order)
        for k in order:
            r, kind, g, per, _ = items[k]
            times.setdefault((r, kind), []).append(time_graph(g, per, 5))
    for r, out in enumerate(rows):
        nbytes = out["bytes_per_set"]
        for kind in ("warm", "cold"):
            t = sorted(times[(r, kind)])
            med, mean = t[len(t) // 2], sum(t) / len(t)
            out[f"{kind}_us"] = round(med, 2)
            out[f"{kind}_us_mean"] = round(mean, 2)
            out[f"{kind}_GBps"] = round(nbytes / (med * 1e-6) / 1e9, 1)
            out[f"{kind}_mean_median_divergence_over_15pct"] = abs(mean - med) > 0.15 * med
        out["cold_frac_of_hbm_peak"] = round(nbytes / (out["cold_us"] * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)
        out["rounds"] = 5
        if oracle_budget_s > 0:
            warm_sets = next(it[4][0] for it in items if it[0] == r and it[1] == "warm")
            spent, done, n, worst, cores = oracle_set(warm_sets[0], out["M"], oracle_budget_s)
            oracle_us = spent / done * nbytes * 1e6
            out["cpu_baseline"] = {
                "kind": "oracle", "us_per_set": round(oracle_us, 1), "GBps": round(done / spent / 1e9, 4),
                "cores": cores, "sample": f"{n} of {out['launches_per_set']} GEMVs, whole, {spent:.2f} s",
                "gpu_speedup_cold": round(oracle_us / out["cold_us"], 1), "host": host_cpu()}
            out["parity_sample"] = {"gemvs_checked": n, "worst_err_over_bound": round(worst, 4),
                                    "ok": bool(worst <= 1.0)}
        print(json.dumps(out), flush=True)
    del items
    torch.cuda.empty_cache()
    return rows


def prefill_gemm(torch, seed, weights):
    """Prefill GEMM timings, M = 2048 on gate+up and down and M = 64 split-K
    on qkv, o and down; weights(layer) gives the packed weights of the 7B
    layer shape of that index. Returns the two JSON sections."""
    # Prefill (M = 2048) on the gate+up and down shapes: the fused W4A16
    # GEMM, the standalone fp16 dequantization, and for context the two-step
    # route (that dequantization, then torch's fp16 library GEMM). Matrix-core
    # runs on this GPU vary by several percent with what ran just before
    # (power and clock state; timed first on a device that had been running
    # only memory-bound work, a GEMM read 5-15% slow), so the three first run
    # under sustained load for a second, then are timed in turn, in a
    # rotating order, five rounds, and each reports its median.
    import int4_weight_only_w4a16_amd as wl
    Mp = 2048

    def timed(fn, reps=10):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    def rotating_rounds(fns, rounds=5, settle_s=1.0):
        """Times of each callable: after settle_s seconds of all of them in
        turn, `rounds` rounds in a rotating order."""
        names = list(fns)
        t_end = time.perf_counter() + settle_s
        while time.perf_counter() < t_end:
            for n in names:
                fns[n]()
            torch.cuda.synchronize()
        runs = {n: [] for n in names}
        for r in range(rounds):
            for n in names[r % len(names):] + names[:r % len(names)]:
                runs[n].append(timed(fns[n]))
        return runs

    prefill = {}
    for label, layer in (("gate_up", 2), ("down", 3)):
        _, Np, Kp = synthetic.QWEN7B_LAYER[layer]
        wq_g, sc_g, zp_g = weights(layer)
        xp = synthetic.device_activations(Mp, Kp, seed, 9999, torch.device("cuda:0"))
        yp = torch.empty((Mp, Np), dtype=torch.int16, device="cuda:0")
        w16 = torch.empty((Np, Kp), dtype=torch.float16, device="cuda:0")
        fns = {"gemm": lambda: wl.w4a16_gemm(Mp, Np, Kp, wq_g, sc_g, zp_g, xp, yp),
               "dq": lambda: wl.w4a16_dequant_f16(Np, Kp, wq_g, sc_g, zp_g, w16),
               "lib": lambda: torch.matmul(xp.view(torch.float16), w16.t())}
        runs = rotating_rounds(fns)
        gemm_us, dq_us, lib_us = (float(np.median(runs[k])) for k in ("gemm", "dq", "lib"))
        flops = 2.0 * Mp * Np * Kp
        dq_bytes = algorithmic_bytes(0, Np, Kp) + 2 * Np * Kp
        prefill[label] = {
            "shape": f"M={Mp} x {label} {Np}x{Kp}",
            "w4a16_gemm_us": round(gemm_us, 1),
            "w4a16_gemm_TFLOPs": round(flops / (gemm_us * 1e-6) / 1e12, 1),
            "w4a16_gemm_frac_of_mfma_f16_peak": round(flops / (gemm_us * 1e-6) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
            "dequant_f16_us": round(dq_us, 1),
            "dequant_f16_GBps": round(dq_bytes / (dq_us * 1e-6) / 1e9, 1),
            "dequant_f16_frac_of_hbm_peak": round(dq_bytes / (dq_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
            "torch_fp16_gemm_us": round(lib_us, 1),
            "two_step_dequant_plus_torch_fp16_gemm_us": round(dq_us + lib_us, 1),
        }
        del xp, yp, w16

    # Short prefill chunks (M = 64, and M = 128 for the narrow matrices)
    # leave the 128 x 128-tile GEMM with a few dozen workgroups on 256 compute
    # units: the split-K GEMM at the split count the library chooses, with
    # the atomic combine and with the two-stage (partials) combine, against
    # the unsplit one and the two-step route, timed in turn as above.
    prefill_small = {}
    for label, layer, Ms in (("qkv", 0, 64), ("o", 1, 64), ("down", 3, 64), ("qkv_m128", 0, 128),
                             ("down_m128", 3, 128)):
        _, Np, Kp = synthetic.QWEN7B_LAYER[layer]
        wq_g, sc_g, zp_g = weights(layer)
        xp = synthetic.device_activations(Ms, Kp, seed, 9998, torch.device("cuda:0"))
        yp = torch.empty((Ms, Np), dtype=torch.int16, device="cuda:0")
        w16 = torch.empty((Np, Kp), dtype=torch.float16, device="cuda:0")
        splits = wl.w4a16_gemm_splitk_choose(Ms, Np, Kp)
        ws_g = torch.zeros(wl.w4a16_splitk_workspace_bytes(Ms, Np, splits), dtype=torch.uint8, device="cuda:0")
        psplits = wl.w4a16_gemm_partials_choose(Ms, Np, Kp)
        part_g = torch.empty(wl.w4a16_gemm_partials_bytes(Ms, Np, psplits), dtype=torch.uint8, device="cuda:0")
        fns = {"gemm": lambda: wl.w4a16_gemm(Ms, Np, Kp, wq_g, sc_g, zp_g, xp, yp),
               "split": lambda: wl.w4a16_gemm_splitk(Ms, Np, Kp, splits, wq_g, sc_g, zp_g, xp, yp, ws_g),
               "partials": lambda: wl.w4a16_gemm_splitk_partials(Ms, Np, Kp, psplits, wq_g, sc_g, zp_g, xp, yp, part_g),
               "dq": lambda: wl.w4a16_dequant_f16(Np, Kp, wq_g, sc_g, zp_g, w16),
               "lib": lambda: torch.matmul(xp.view(torch.float16), w16.t())}
        runs = rotating_rounds(fns)
        gemm_us, split_us, part_us, dq_us, lib_us = (float(np.median(runs[k]))
                                                     for k in ("gemm", "split", "partials", "dq", "lib"))
        prefill_small[label] = {
            "shape": f"M={Ms} x {label.split('_')[0]} {Np}x{Kp}",
            "splits": splits,
            "w4a16_gemm_splitk_us": round(split_us, 1),
            "partials_splits": psplits,
            "w4a16_gemm_splitk_partials_us": round(part_us, 1),
            "w4a16_gemm_unsplit_us": round(gemm_us, 1),
            "two_step_dequant_plus_torch_fp16_gemm_us": round(dq_us + lib_us, 1),
            "splitk_TFLOPs": round(2.0 * Ms * Np * Kp / (split_us * 1e-6) / 1e12, 1),
            "splitk_weight_GBps": round(algorithmic_bytes(0, Np, Kp) / (split_us * 1e-6) / 1e9, 1),
        }
        del xp, yp, w16, ws_g, part_g

    return prefill, prefill_small


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--roofline-reps", type=int, default=100)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of oracle time (0: skip)")
    ap.add_argument("--trace-summary", metavar="DIR")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 512 MiB device copy kernel (counter scaling)")
    ap.add_argument("--configs", action="store_true",
                    help="time every workload configuration warm and cold (one JSON line each) instead")
    ap.add_argument("--counter-pass", action="store_true",
                    help="launch each counter-pass shape a few times (for a rocprofv3 --pmc run)")
    ap.add_argument("--counter-summary", nargs="+", metavar="DIR",
                    help="summarize counter-pass rocprofv3 runs (one directory per counter set)")
    ap.add_argument("--decompose", type=int, metavar="STEPS",
                    help="trace STEPS graph and STEPS eager steps (for rocprofv3 --kernel-trace), then time both")
    ap.add_argument("--decompose-summary", metavar="DIR", help="step decomposition from a --decompose trace")
    ap.add_argument("--gemm-counter-summary", nargs="+", metavar="DIR",
                    help="summarize rocprofv3 --pmc runs of --prefill-gemm (one directory per counter set)")
    ap.add_argument("--prefill-gemm", action="store_true",
                    help="time only the prefill GEMM section (for counter passes) and print it as one JSON line")
    ap.add_argument("--read-floor", action="store_true",
                    help="time a plain read of each 7B GEMV's bytes against the GEMV (graph, cold) instead")
    args = ap.parse_args()

    if args.trace_summary:
        trace_summary(args.trace_summary)
        return
    if args.counter_summary:
        counter_summary(args.counter_summary)
        return
    if args.decompose_summary:
        decompose_summary(args.decompose_summary, args.decompose or 20)
        return
    if args.gemm_counter_summary:
        gemm_counter_summary(args.gemm_counter_summary)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the W4A16 GEMV path here is single-GPU "
              "(--gpus 1 only).", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        n = (512 << 20) // 4
        a = torch.ones(n, dtype=torch.int32, device="cuda:0")
        b = torch.empty_like(a)
        for _ in range(3):
            torch.neg(a, out=b)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "launches": 3}))
        return

    if args.configs:
        run_configs(torch, args.seed)
        return
    if args.counter_pass:
        counter_pass(torch, args.seed)
        return
    if args.decompose:
        decompose_pass(torch, args.seed, args.decompose)
        return
    if args.read_floor:
        read_floor(torch, args.seed)
        return
    if args.prefill_gemm:
        dev = torch.device("cuda:0")
        pre, small = prefill_gemm(torch, args.seed, lambda layer: synthetic.device_packed_weights(
            synthetic.QWEN7B_LAYER[layer][1], synthetic.QWEN7B_LAYER[layer][2], args.seed, layer, dev))
        print(json.dumps({"prefill_gemm": pre, "prefill_gemm_small_m": small}), flush=True)
        return

    t_setup = time.perf_counter()
    step = Step(args.seed, torch)
    graph = step.capture()
    setup_s = time.perf_counter() - t_setup

    elapsed = step.time_graph(graph, args.steps, args.warmup)
    us_step = elapsed / args.steps * 1e6
    value = step.bytes * args.steps / elapsed / 1e9
    eager_us = step.time_eager(max(3, args.steps // 10)) / max(3, args.steps // 10) * 1e6

    def median_rounds(g, reps, rounds=5):
        """Median over `rounds` timings of `reps` replays, after one untimed
        pass of as many, so that no single round (the first after the eager
        timing, which leaves the device idle between launches, say) sets the
        figure. Returns (median, fastest, slowest) in seconds."""
        step.time_graph(g, reps, 3)
        t = sorted(step.time_graph(g, reps, 3) for _ in range(rounds))
        return t[len(t) // 2], t[0], t[-1]

    # Dominant kernel: the gate+up GEMV (58% of the step's bytes), 28 distinct
    # weight sets back to back in one graph.
    dom = step.capture(only="gate_up_proj")
    reps = args.roofline_reps
    dom_s, dom_fast_s, dom_slow_s = median_rounds(dom, reps)
    n_dom = synthetic.QWEN7B_LAYERS
    _, Nd, Kd = synthetic.QWEN7B_LAYER[2]
    dom_bytes = algorithmic_bytes(1, Nd, Kd)
    dom_us = dom_s / (reps * n_dom) * 1e6
    achieved = dom_bytes / (dom_us * 1e-6) / 1e9

    read_ceiling = read_ceiling_gbps(torch)

    # Variant (reported beside, never as `value`): gate+up with the SwiGLU
    # epilogue fused, y = silu(g) * u of width 18944, same weight bytes.
    fused = step.capture(only="gate_up_proj", swiglu=True)
    fused_s = median_rounds(fused, reps)[0]
    fused_us = fused_s / (reps * n_dom) * 1e6
    fused_bytes = dom_bytes - 2 * Nd + 2 * (Nd // 2)
    fused_step = step.capture(swiglu=True)
    fused_step_s = step.time_graph(fused_step, args.steps, args.warmup)
    unfused = step.capture(only="gate_up_proj", torch_act=True)
    unfused_us = median_rounds(unfused, reps)[0] / (reps * n_dom) * 1e6
    del fused, fused_step, unfused

    # Variant: INT8 activations (the dp4a path of the H100 runtime page, here
    # on the integer matrix cores): a quantize launch before each GEMV.
    a8_gate_up = step.capture(only="gate_up_proj", a8="both")
    a8_gate_up_us = median_rounds(a8_gate_up, reps)[0] / (reps * n_dom) * 1e6
    a8_gemv = step.capture(only="gate_up_proj", a8="gemv")
    a8_gemv_us = median_rounds(a8_gemv, reps)[0] / (reps * n_dom) * 1e6
    a8_step = step.capture(a8="both")
    a8_step_us = step.time_graph(a8_step, args.steps, args.warmup) / args.steps * 1e6
    # The quantization fused into the GEMV: one launch per GEMV again.
    a8f_gate_up = step.capture(only="gate_up_proj", a8="fused")
    a8f_gate_up_us = median_rounds(a8f_gate_up, reps)[0] / (reps * n_dom) * 1e6
    a8f_step = step.capture(a8="fused")
    a8f_step_us = step.time_graph(a8f_step, args.steps, args.warmup) / args.steps * 1e6
    del a8_gate_up, a8_gemv, a8_step, a8f_gate_up, a8f_step

    prefill, prefill_small = prefill_gemm(torch, args.seed, lambda layer: step.bufs[layer][3:6])
    import int4_weight_only_w4a16_amd as wl

    # Host quantizer (w4a16_quantize) on the qkv matrix's shape: fp16 in.
    wlib = wl
    _, Nq, Kq = synthetic.QWEN7B_LAYER[0]
    wq16 = (np.random.default_rng(args.seed).standard_normal((Nq, Kq)) * 0.02).astype(np.float16)
    quant = {}
    for mode, label in ((0, "symmetric"), (1, "asymmetric")):
        wlib.w4a16_quantize(wq16, mode)  # warm
        t0 = time.perf_counter()
        wlib.w4a16_quantize(wq16, mode)
        quant[label] = round(wq16.nbytes / (time.perf_counter() - t0) / 1e9, 3)

    # The whole step as one persistent launch, beside the graph of 113.
    chain = ChainStep(step, torch)
    chain_s = chain.time(args.steps, args.warmup)
    chain_err = chain.error_word()  # sticky: nonzero would mean every timed run returned at once
    chain_ys = chain.outputs()
    chain_out = {
        "kernel": "w4a16_chain_run: the step's 113 GEMVs in one persistent launch, each fed by its producer "
                  "(tagged handoff words), two resident 8-wave workgroups per CU",
        "us_per_step": round(chain_s * 1e6, 2),
        "graph_us_per_step": round(us_step, 2),
        "ratio_to_graph": round(chain_s * 1e6 / us_step, 3),
        "GBps": round(step.bytes / chain_s / 1e9, 1),
        "launches_per_step": 1,
        "down_splits": 1,
        "error_word": chain_err,
        "handoff": handoff_costs(torch, args.seed),
    }

    # Outputs of the last full replay, for the sampled check.
    graph.replay()
    torch.cuda.synchronize()

    out = {
        "metric": "achieved HBM GB/s for batch-1 W4A16 GEMV over a 7B decode step (us per step in ms_per_step)",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us_step / 1e3, 5),
        "us_per_step": round(us_step, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4 x fp16 -> fp32",
        "data": "synthetic (seeded; packed int4 weights, fp16 scales |N(0,0.02)|+1e-3, uniform 4-bit zeros, x ~ N(0,1))",
        "config": {
            "workload": "Qwen2.5-7B-shaped decode step at M=1: 28 x (qkv 4608x3584, o 3584x3584, "
                        "gate_up 37888x3584, down 3584x18944) + lm_head 152064x3584, int4 g=128",
            "launches_per_step": len(step.shapes),
            "bytes_per_step": step.bytes,
            "submission": "one captured graph per step",
            "split_k": {f"{N}x{K}": sp for (N, K), sp in step.splits.items() if sp > 1},
            "eager_us_per_step": round(eager_us, 1),
            "frac_of_hbm_peak": round(value / HBM_PEAK_GBPS, 4),
            "frac_of_measured_read_ceiling": round(value / read_ceiling, 4),
        },
        "roofline": {
            "kernel": "w4a16 gemv, gate_up 37888x3584 M=1",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": load_traffic(),
            "bytes_per_launch": dom_bytes,
            "avg_launch_us": round(dom_us, 3),
            "avg_launch_us_fastest_slowest_round": [round(dom_fast_s / (reps * n_dom) * 1e6, 3),
                                                    round(dom_slow_s / (reps * n_dom) * 1e6, 3)],
            "measured_read_ceiling_GBps": round(read_ceiling, 1),
            "frac_of_measured_read_ceiling": round(achieved / read_ceiling, 4),
        },
        "variants": {
            "gate_up_swiglu_fused": {
                "kernel": "w4a16_gemv_swiglu, gate+up 37888x3584 -> silu(g)*u 18944, M=1",
                "avg_launch_us": round(fused_us, 3),
                "achieved_GBps": round(fused_bytes / (fused_us * 1e-6) / 1e9, 1),
                "frac": round(fused_bytes / (fused_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                "bytes_per_launch": fused_bytes,
                "plain_gate_up_us": round(dom_us, 3),
                "unfused_gate_up_plus_torch_silu_mul_us": round(unfused_us, 3),
                "step_us_with_fused_gate_up": round(fused_step_s / args.steps * 1e6, 2),
            },
        },
        "int8_activations": {
            "kernels": "w4a16_act_quant_i8 + w4a16_gemv_a8 (v_mfma_i32_16x16x64_i8), per GEMV",
            "gate_up_quant_plus_gemv_us": round(a8_gate_up_us, 3),
            "gate_up_gemv_a8_only_us": round(a8_gemv_us, 3),
            "gate_up_fp16_activations_us": round(dom_us, 3),
            "step_us": round(a8_step_us, 2),
            "step_us_fp16_activations": round(us_step, 2),
            "launches_per_step": 2 * len(step.shapes),
            "fused": {
                "kernel": "w4a16_gemv_a8_fused (quantization inside the GEMV launch, bit-identical)",
                "gate_up_us": round(a8f_gate_up_us, 3),
                "step_us": round(a8f_step_us, 2),
                "launches_per_step": len(step.shapes),
            },
        },
        "chain": chain_out,
        "prefill_gemm": prefill,
        "prefill_gemm_small_m": prefill_small,
        "host_quantize": {"shape": f"{Nq}x{Kq} fp16", "GBps_fp16_in": quant,
                          "threads": os.cpu_count()},
        "setup_s": round(setup_s, 1),
    }
    if args.cpu_budget > 0:
        cpu, worst, n_checked = cpu_baseline(step, args.cpu_budget)
        out["cpu_baseline"] = cpu
        out["parity_sample"] = {"gemvs_checked": n_checked, "worst_err_over_bound": round(worst, 4),
                                "ok": bool(worst <= 1.0)}
        c_worst, c_checked = check_chain(chain, chain_ys)
        out["chain"]["parity"] = {"gemvs_checked": c_checked, "worst_err_over_bound": round(c_worst, 4),
                                  "ok": bool(c_worst <= 1.0)}
    print(json.dumps(out))


if __name__ == "__main__":
    main()
