#!/usr/bin/env python3
"""Benchmark of the ternary-weight x int8-activation hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--tokens N] [--no-graph] [--no-cpu] [--no-extra]

A step is one pass of the whole path over one batch: for every layer, each of
the four projection groups quantizes its input per token (absmax int8) and
runs its ternary products with the fused dequantization epilogue (through the
per-layer driver: at one token a single launch per layer does all of it).  Weights
are packed once at load time (not timed; timed separately as "pack").
Inputs already sit in HBM when the timed region starts.

Default workload: the 80-layer 70B-class weight stream (hidden 8192, FFN
28672, 64 q / 8 kv heads; 17.1 GB of packed ternary weights) at 1 token.  It
is the largest single-GPU workload and the only one whose weights cannot sit
in the 256 MB last-level cache, so its packed-weight GB/s is an HBM figure.
The same line also reports the 8-token stream and the 2048-token prefill of
the 2B-class block (int8 TOPS), under "extra".

Prints ONE JSON line (the metric: packed-weight GB/s and fraction of HBM peak
for decode; int8 TOPS and fraction of the int8 matrix-core peak for prefill).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("packed-weight GB/s & % HBM peak (decode GEMV); "
          "int8 TOPS & % MFMA peak (prefill)")
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, published
PEAK_INT8_TOPS = 5000.0      # MI355X dense int8 matrix cores, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
TRACE_FILE = os.path.join(ROOT, "profiles", "kernel_trace.json")
# Sources of each measured kernel: a traffic record is only used while they
# are unchanged since the counters were taken.
KERNEL_SOURCES = {
    "layer_dot4_kernel": ("layer.hip", "layer.hpp", "dot4.hpp", "base3.hpp", "common.hpp",
                          "quant.hpp", "internal.hpp"),
    "decode_dot4_kernel (fused quantization)": ("gemv.hip", "dot4.hpp", "common.hpp", "group.hpp",
                                                "quant.hpp"),
    "decode_dot4_kernel": ("gemv.hip", "dot4.hpp", "common.hpp", "group.hpp", "quant.hpp"),
    "decode_mfma_kernel": ("mfma.hip", "common.hpp", "group.hpp"),
    "prefill_kernel": ("prefill.hip", "common.hpp", "group.hpp"),
    "prefill_multi_kernel": ("prefill.hip", "common.hpp", "group.hpp", "quant.hip", "quant.hpp"),
    "decode_mfma_multi_kernel": ("mfma.hip", "common.hpp", "group.hpp", "quant.hip", "quant.hpp"),
}
# Steps of the prefill extra (at least these many, whatever --steps and
# --warmup say; multiples of its 20 steps per graph).
PREFILL_MIN_STEPS, PREFILL_MIN_WARMUP, PREFILL_PER_GRAPH = 200, 2000, 20


def prefill_steps(steps, warmup):
    g = PREFILL_PER_GRAPH
    return max(steps, PREFILL_MIN_STEPS) // g * g, max(warmup, PREFILL_MIN_WARMUP) // g * g


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=50,
                    help="untimed steps before the timed ones (the default, ~0.2 s of "
                         "the 70B-class stream, lets the chip reach its steady clocks)")
    ap.add_argument("--workload", default="stream70b")
    ap.add_argument("--tokens", type=int, default=None,
                    help="tokens per step (default: the workload's first batch)")
    ap.add_argument("--layers", type=int, default=None,
                    help="override the number of layers (default: the workload's)")
    ap.add_argument("--no-graph", action="store_true",
                    help="launch the step eagerly instead of replaying a HIP graph")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the 8-token stream and the prefill extras")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a device-to-device copy of 1 GiB, five times "
                         "(reference for the HBM traffic counters)")
    ap.add_argument("--base3-only", action="store_true",
                    help="only compare the 2-bit and base-3 weight formats on the "
                         "70B-class matrices (--layers blocks deep, default 8)")
    ap.add_argument("--trace-summary", metavar="DIR",
                    help="no GPU: read the rocprofv3 --kernel-trace csv output of a "
                         "default-workload bench run made with the same --steps / "
                         "--warmup / --layers, keep the per-layer kernel's dispatches "
                         "of the timed steps only, and rewrite its entry of "
                         "profiles/kernel_trace.json")
    ap.add_argument("--traffic-summary", nargs=4, metavar="DIR",
                    help="no GPU: read four rocprofv3 --pmc output folders (copy "
                         "FETCH_SIZE, copy WRITE_SIZE, step FETCH_SIZE, step "
                         "WRITE_SIZE) and rewrite the layer kernel's entry of "
                         "profiles/traffic.json")
    return ap.parse_args()


def note(msg: str):
    """A progress line on stderr (the JSON result is the only stdout line)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_sha(kernel_name: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel_name]:
        with open(os.path.join(ROOT, "ternary_weight_quantized_bt_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


class Model:
    """Packed weights of every layer plus per-step inputs, outputs, workspace."""

    def __init__(self, wl, layers, device, base3=False):
        import torch
        import ternary_weight_quantized_bt_amd as bt
        import workloads as W
        self.wl, self.layers, self.device = wl, layers, device
        self.layer_objs = []
        t0 = time.perf_counter()
        pack_s = 0.0
        for l in range(layers):
            packed = []
            for p, (M, K) in enumerate(wl.shapes):
                w = W.ternary_weights(M, K, wl.weight_dist, W.weight_seed(wl, l, p), device)
                torch.cuda.synchronize()
                a = time.perf_counter()
                packed.append(bt.pack_b3(w, W.weight_scale(wl, p)) if base3
                              else bt.pack(w, W.weight_scale(wl, p)))
                torch.cuda.synchronize()
                pack_s += time.perf_counter() - a
                del w
            self.layer_objs.append(bt.Layer(packed, wl.shapes, base3=base3))
        self.setup_s = time.perf_counter() - t0
        self.pack_s = pack_s
        self.packed_bytes = (sum(t.numel() - 256 for t in self.layer_objs[0].packed) * layers
                             if base3 else wl.packed_bytes_per_layer * layers)

    def set_tokens(self, N):
        import torch
        import ternary_weight_quantized_bt_amd as bt
        import workloads as W
        wl = self.wl
        self.N = N
        ydt = bt.BT_BF16 if wl.y_dtype == "bf16" else bt.BT_F32
        self.ydt = ydt
        self.xs = [W.layer_inputs(wl, l, N, self.device) for l in range(self.layers)]
        L0 = self.layer_objs[0]
        self.ws = L0.alloc_workspace(N, self.device)
        self.ys = [L.alloc_outputs(N, ydt, self.device) for L in self.layer_objs]
        self.ios = [L.make_io(x, y, ydt, self.ws)
                    for L, x, y in zip(self.layer_objs, self.xs, self.ys)]
        self.ios_pg = [L.make_io(x, y, ydt, self.ws, per_group=True)
                       for L, x, y in zip(self.layer_objs, self.xs, self.ys)]
        xdt = bt.BT_BF16 if wl.x_dtype == "bf16" else bt.BT_F32
        self.one_launch = bt.bt_layer_one_launch(L0.c, N, xdt) == 1
        # quantized copies of every input, for the kernel-only timing pass
        self.q = [[bt.quant_act(x) for x in xs] for xs in self.xs]
        self.groups = []
        first = (0, 3, 4, 6)
        count = (3, 1, 2, 1)
        for l, L in enumerate(self.layer_objs):
            gl = []
            for i in range(4):
                items = [(L.packed[p], wl.shapes[p][0], self.ys[l][p])
                         for p in range(first[i], first[i] + count[i])]
                gl.append((bt.make_projs(items), count[i], wl.shapes[first[i]][1], i))
            self.groups.append(gl)
        torch.cuda.synchronize()

    def step(self):
        import ternary_weight_quantized_bt_amd as bt
        for L, io in zip(self.layer_objs, self.ios):
            bt.bt_layer_forward(L.c, io)

    def step_per_group(self):
        """The same step with every layer run as four group launches."""
        import ternary_weight_quantized_bt_amd as bt
        for L, io in zip(self.layer_objs, self.ios_pg):
            bt.bt_layer_forward(L.c, io)

    def products_only(self):
        """The step's grouped product launches, back to back, on inputs that
        are already quantized (same kernels and grids as in the step)."""
        import ternary_weight_quantized_bt_amd as bt
        for l, gl in enumerate(self.groups):
            for projs, count, K, i in gl:
                xq, xs, xsum = self.q[l][i]
                bt.bt_ternary_matmul_group(projs, count, K, xq, xs, xsum, self.N, self.ydt)


def time_region(fn, reps):
    import torch
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for _ in range(reps):
        fn()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(end) / 1e3, wall


def run_steps(model, steps, warmup, use_graph, step=None, per_graph=1):
    """Returns (seconds per step, wall seconds of the timed region).

    With a graph, `per_graph` consecutive steps are captured in one graph and
    the graph is replayed steps / per_graph times (every step still runs in
    full; only the host's per-replay launch cost is shared, as when a graph
    holds a whole model's blocks)."""
    import torch
    step = step or model.step
    if use_graph:
        if steps % per_graph or warmup % per_graph:
            raise ValueError("steps and warmup must be multiples of per_graph")
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            step()  # eager warm-up on the capture stream
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for _ in range(per_graph):
                step()
        fn = g.replay
    else:
        fn, per_graph = step, 1
    for _ in range(warmup // per_graph):
        fn()
    t, wall = time_region(fn, steps // per_graph)
    return t / steps, wall


def kernel_pass(model, reps):
    """Average duration of the dominant kernel's launches (HIP events around
    back-to-back runs of every grouped product of a step)."""
    model.products_only()
    t, _ = time_region(model.products_only, reps)
    launches = 4 * model.layers * reps
    return t / launches, launches


def read_traffic(kernel_name, sha):
    try:
        with open(TRAFFIC_FILE) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    e = d.get(kernel_name)
    if not e or e.get("kernel_sha") != sha:
        return None
    return e.get("bytes_per_launch")


def _pmc_rows(folder, counter):
    """(kernel name, counter value) of every dispatch in a rocprofv3 --pmc
    csv output folder."""
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(folder, "*counter_collection.csv")):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter:
                    rows.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return rows


def traffic_summary(copy_fetch, copy_write, k_fetch, k_write):
    """HBM bytes per launch of the layer kernel from FETCH_SIZE / WRITE_SIZE
    (KiB per dispatch), each scaled by what the counter reads for a 1 GiB
    device copy (the copy reads and writes 2^30 bytes)."""
    name = "layer_dot4_kernel"
    copy = (1 << 30) / 1024.0

    def mean(rows, key):
        v = [x for k, x in rows if key in k]
        if not v:
            raise SystemExit(f"no {key} dispatches found")
        return sum(v) / len(v), len(v)

    cf, _ = mean(_pmc_rows(copy_fetch, "FETCH_SIZE"), "copyBuffer")
    cw, _ = mean(_pmc_rows(copy_write, "WRITE_SIZE"), "copyBuffer")
    kf, n = mean(_pmc_rows(k_fetch, "FETCH_SIZE"), name)
    kw, _ = mean(_pmc_rows(k_write, "WRITE_SIZE"), name)
    rf, rw = copy / cf, copy / cw
    read, write = kf * 1024 * rf, kw * 1024 * rw
    alg = _block_packed_bytes()
    entry = {
        "kernel_sha": kernel_sha(name),
        "bytes_per_launch": int(round(read + write)),
        "read_bytes_per_launch": int(round(read)),
        "write_bytes_per_launch": int(round(write)),
        "algorithmic_bytes_per_launch": alg,
        "read_over_algorithmic": round(read / alg, 4),
        "calibration": f"1 GiB device copy: FETCH_SIZE {cf:.1f} KiB (read factor {rf:.5f}), "
                       f"WRITE_SIZE {cw:.0f} KiB (write factor {rw:.4f})",
        "workload": "stream70b, 1 token, one launch per layer",
        "dispatches": n,
    }
    try:
        with open(TRAFFIC_FILE) as f:
            d = json.load(f)
    except (OSError, ValueError):
        d = {}
    d[name] = entry
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(d, f, indent=1)
    print(json.dumps(entry, indent=1))


def _trace_rows(folder):
    """(kernel name, start ns, end ns) of every dispatch in a rocprofv3
    --kernel-trace csv output folder, in start order."""
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(folder, "**", "*kernel_trace.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                rows.append((r["Kernel_Name"], int(r["Start_Timestamp"]),
                             int(r["End_Timestamp"])))
    rows.sort(key=lambda r: r[1])
    return rows


def _headline_kernel(name):
    """The one-token per-layer kernel on T16Q256 weights (template arguments
    <element type, tokens, waves, K split, ring, base-3>)."""
    if "layer_dot4_kernel<" not in name:
        return False
    args = [a.strip() for a in name.split("layer_dot4_kernel<", 1)[1].split(">", 1)[0].split(",")]
    return len(args) == 6 and args[1] == "1" and args[5] == "false"


def trace_summary(folder, steps, warmup, layers, out=TRACE_FILE):
    """Durations of the per-layer kernel's dispatches inside the timed window
    of a bench run: the run's first `layers` dispatches of it are the eager
    step before the graph capture, the next warmup * layers the untimed graph
    replays, the next steps * layers the timed replays."""
    import statistics
    name = "layer_dot4_kernel"
    rows = [r for r in _trace_rows(folder) if _headline_kernel(r[0])]
    skip, count = layers * (1 + warmup), layers * steps
    if len(rows) < skip + count:
        raise SystemExit(f"{len(rows)} dispatches of the kernel, need {skip + count}")
    win = rows[skip:skip + count]
    d = [(e - b) / 1e3 for _, b, e in win]
    span = (win[-1][2] - win[0][1]) / 1e3
    entry = {
        "kernel_sha": kernel_sha(name),
        "kernel_instance": win[0][0],
        "timed_dispatches": count,
        "mean_us": round(statistics.fmean(d), 3),
        "median_us": round(statistics.median(d), 3),
        "min_us": round(min(d), 3),
        "max_us": round(max(d), 3),
        "window_span_ms": round(span / 1e3, 4),
        "span_per_step_ms": round(span / steps / 1e3, 4),
        "busy_fraction_of_span": round(sum(d) / span, 4),
        "steps": steps, "warmup": warmup, "layers": layers,
        "skipped_dispatches": skip,
    }
    try:
        with open(out) as f:
            doc = json.load(f)
    except (OSError, ValueError):
        doc = {}
    doc[name] = entry
    # The grouped launches of the 8-token stream and of the 2048-token
    # prefill, each with the quantization launch just before it: the timed
    # window of each (its first eager step and warm-up replays skipped).
    all_rows = _trace_rows(folder)
    psteps, pwarm = prefill_steps(steps, warmup)
    for key, marker, skip_n, count_n in (
            ("decode_mfma_multi_kernel", "decode_mfma_multi_kernel<", layers * (1 + warmup),
             layers * steps),
            ("prefill_multi_kernel", "prefill_multi_kernel<", 1 + pwarm, psteps)):
        g = _grouped_window(all_rows, marker, skip_n, count_n)
        if g is not None:
            g["kernel_sha"] = kernel_sha(key)
            doc[key] = g
    with open(out, "w") as f:
        json.dump(doc, f, indent=1)
    print(json.dumps(entry, indent=1))
    return entry


def _grouped_window(rows, marker, skip, count):
    """Mean durations of a grouped product kernel's dispatches [skip, skip +
    count) (in start order) and of the quantization launch that precedes each
    one, with the mean and median gap between the two; None if the trace has
    fewer."""
    import statistics
    idx = [i for i, r in enumerate(rows) if marker in r[0]]
    if len(idx) < skip + count:
        return None
    win = idx[skip:skip + count]
    prod = [(rows[i][2] - rows[i][1]) / 1e3 for i in win]
    quant, gap = [], []
    for i in win:
        j = i - 1
        while j >= 0 and "quant_onepass_kernel<" not in rows[j][0]:
            j -= 1
        if j >= 0:
            quant.append((rows[j][2] - rows[j][1]) / 1e3)
            gap.append((rows[i][1] - rows[j][2]) / 1e3)
    out = {"kernel_instance": rows[win[0]][0], "timed_dispatches": count,
           "skipped_dispatches": skip, "mean_us": round(statistics.fmean(prod), 3),
           "median_us": round(statistics.median(prod), 3), "min_us": round(min(prod), 3)}
    if quant:
        out["quant_mean_us"] = round(statistics.fmean(quant), 3)
        out["quant_to_product_gap_mean_us"] = round(statistics.fmean(gap), 3)
        # the tracer's timestamps occasionally pair a product with an
        # overlapping or distant quantization record; the median is robust
        out["quant_to_product_gap_median_us"] = round(statistics.median(gap), 3)
    return out


def read_trace(kernel_name, sha):
    try:
        with open(TRACE_FILE) as f:
            e = json.load(f).get(kernel_name)
    except (OSError, ValueError):
        return None
    return e if e and e.get("kernel_sha") == sha else None


def _block_packed_bytes():
    """Packed code bytes of one 70B-class block (the seven projections)."""
    import workloads as W
    return W.STREAM70B.packed_bytes_per_layer


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def _repeat(fn, budget_s):
    """Calls fn until budget_s have passed (at least once): (calls, seconds)."""
    reps, t0 = 0, time.perf_counter()
    while True:
        fn()
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            return reps, el


def _oracle_layer(wl, N, rows_per_proj=None):
    """The oracle's whole path on layer 0 of a workload (the same seeded
    weights and inputs as the GPU): per projection, quantize its input, the
    exact product (all rows, or a fixed sample of rows), dequantization.
    Returns (callable, packed bytes it streams, int8 ops it performs)."""
    import numpy as np
    import torch
    import oracle
    import workloads as W
    dev = "cuda:0"
    packed, rows = [], []
    for p, (M, K) in enumerate(wl.shapes):
        w = W.ternary_weights(M, K, wl.weight_dist, W.weight_seed(wl, 0, p), dev).cpu().numpy()
        packed.append(oracle.pack(w, W.weight_scale(wl, p))[0])
        del w
        rows.append(None if rows_per_proj is None else
                    np.linspace(0, M - 1, rows_per_proj).astype(np.int64))
    xs = W.layer_inputs(wl, 0, N, dev)
    xs = [x.cpu().view(torch.uint16).numpy() if x.dtype == torch.bfloat16
          else x.cpu().numpy() for x in xs]

    def run():
        for p, (M, K) in enumerate(wl.shapes):
            xq, xsc, _ = oracle.quant_act(xs[wl.proj_input[p]])
            acc = oracle.matmul_i32(packed[p], M, K, xq, rows[p])
            oracle.dequant(acc, oracle.scale_of(packed[p], M, K), xsc)
    nrow = [M if r is None else len(r) for (M, _), r in zip(wl.shapes, rows)]
    streamed = sum(n * K // 4 for n, (_, K) in zip(nrow, wl.shapes))
    ops = 2 * N * sum(n * K for n, (_, K) in zip(nrow, wl.shapes))
    return run, streamed, ops


def _threads(n):
    """Sets the oracle's OpenMP thread count (its results do not depend on
    it); returns False if the runtime cannot be reached."""
    try:
        import ctypes
        ctypes.CDLL("libgomp.so.1").omp_set_num_threads(n)
        return True
    except OSError:
        return False


def cpu_baseline(wl, N, budget_s):
    """The oracle on layer 0 of the benchmarked workload (all seven
    projections, the same seeded weights and inputs), repeated until the time
    budget is used, on the host's threads and then on one thread; and the
    same for the four smaller workloads (single GEMV, 2B-style block at 1 and
    64 tokens, the 2048-token prefill on a fixed sample of output rows)."""
    import oracle
    import workloads as W
    cores = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
    cores = min(cores, len(os.sched_getaffinity(0)))
    run, streamed, _ = _oracle_layer(wl, N)
    reps, el = _repeat(run, budget_s)
    one = None
    if _threads(1):
        reps1, el1 = _repeat(run, budget_s / 4)
        _threads(cores)
        one = round(streamed * reps1 / el1 / 1e9, 4)
    per_config = {}
    for cwl, cN, rows, label in (
            (W.GEMV_2560, 1, None, "quantization + product + dequantization, all rows"),
            (W.LAYER2B_N1, 1, None, "7 projections, all rows"),
            (W.LAYER2B_N64, 64, None, "7 projections, all rows"),
            (W.PREFILL2B_N2048, 2048, 32,
             "7 projections, all 2048 tokens quantized, products on 32 evenly spaced "
             "rows per projection")):
        crun, cbytes, cops = _oracle_layer(cwl, cN, rows)
        entry = {"tokens": cN, "sample": label}
        for name, threads, budget in (("threads", cores, 2.0), ("one_thread", 1, 1.0)):
            if threads == 1 and not _threads(1):
                continue
            r, t = _repeat(crun, budget)
            entry[name] = {"calls": r, "seconds": round(t, 2),
                           "ms_per_call": round(t / r * 1e3, 3),
                           "packed_gb_per_s": round(cbytes * r / t / 1e9, 4),
                           "int8_tops": round(cops * r / t / 1e12, 6)}
        _threads(cores)
        per_config[cwl.name] = entry
    return {
        "value": round(streamed * reps / el / 1e9, 4),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"layer 0 of {wl.name} (all 7 projections, {N} token(s)), "
                  f"{reps} pass(es) in {el:.1f} s",
        "one_thread_value": one,
        "cpu_model": _cpu_model(),
        "compile_flags": " ".join(oracle.CFLAGS),
        "per_config": per_config,
    }


def prefill_extra(steps, warmup, use_graph):
    import torch
    import workloads as W
    wl = W.PREFILL2B_N2048
    m = Model(wl, 1, "cuda:0")
    m.set_tokens(2048)
    # one block per step: 20 steps per graph (a model's graph holds its 30
    # blocks), so one replay launch is not charged to every block.  A step is
    # only ~0.15 ms: at least 2000 warm-up steps (~0.3 s) bring the chip to
    # its steady clocks, and at least 200 timed steps average out the noise.
    steps, pwarm = prefill_steps(steps, warmup)
    sec, _ = run_steps(m, steps, pwarm, use_graph, per_graph=PREFILL_PER_GRAPH)
    ops = 2 * 2048 * sum(M * K for M, K in wl.shapes)
    kt, launches = kernel_pass(m, steps)
    res = {
        "workload": wl.name, "tokens": 2048, "ms_per_step": round(sec * 1e3, 4),
        "int8_tops": round(ops / sec / 1e12, 2),
        "frac_of_int8_peak": round(ops / sec / 1e12 / PEAK_INT8_TOPS, 4),
        # the four group products as separate launches, back to back, on
        # inputs quantized beforehand (the step runs them as one launch)
        "per_group_launches_us": round(4 * kt * 1e6, 2),
        "per_group_launches_tops": round(ops / (4 * kt) / 1e12, 2),
    }
    # The step's four-group product launch alone, from a rocprofv3 kernel
    # trace of this command (timed window), while its sources are unchanged.
    tr = read_trace("prefill_multi_kernel", kernel_sha("prefill_multi_kernel"))
    if tr:
        res["rocprof_product_kernel_us"] = tr["mean_us"]
        res["rocprof_product_kernel_tops"] = round(ops / (tr["mean_us"] * 1e-6) / 1e12, 2)
        res["rocprof_product_frac_of_int8_peak"] = round(
            ops / (tr["mean_us"] * 1e-6) / 1e12 / PEAK_INT8_TOPS, 4)
        if "quant_mean_us" in tr:
            res["rocprof_quant_kernel_us"] = tr["quant_mean_us"]
    del m
    torch.cuda.empty_cache()
    return res


def weight_quant_extra(steps, warmup):
    """The float -> ternary weight quantizer on one 28672 x 8192 bf16 matrix
    (the gate / up shape of the 70B-class block), both scale modes.  Bytes
    are those the passes must move: the weights read once per pass (max,
    exact sum for AbsMean, pack) and the packed matrix written."""
    import torch
    import ternary_weight_quantized_bt_amd as bt
    import workloads as W
    M, K = 28672, 8192
    dev = "cuda:0"
    w = W.float_weights(M, K, "normal", 77, "bf16", device=dev)
    packed = torch.empty(bt.bt_packed_bytes(M, K), dtype=torch.uint8, device=dev)
    stats = torch.empty(2, dtype=torch.float32, device=dev)
    wsb = bt.bt_quantize_weights_workspace_bytes()
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    res = {"shape": [M, K], "dtype": "bf16"}
    for name, mode, passes in (("absmean", bt.BT_WSCALE_ABSMEAN, 3),
                               ("absmax", bt.BT_WSCALE_ABSMAX, 2)):
        def call():
            bt.bt_quantize_weights(w, bt.BT_BF16, M, K, mode, 1e-5, packed, stats, ws, wsb)
        for _ in range(warmup):
            call()
        t, _ = time_region(call, steps)
        t /= steps
        moved = passes * M * K * 2 + packed.numel()
        res[name] = {"ms": round(t * 1e3, 4),
                     "weights_gb_per_s": round(M * K * 2 / t / 1e9, 1),
                     "moved_gb_per_s": round(moved / t / 1e9, 1),
                     "frac_of_hbm_peak": round(moved / t / 1e9 / PEAK_HBM_GBS, 4)}
    del w, packed
    torch.cuda.empty_cache()
    return res


def base3_stream_extra(wl, layers, steps, warmup, use_graph, value_2bit, sec_2bit):
    """The same 1-token stream with the weights in the base-3 B3T1024 format
    (1.625 bits per weight): one launch per block, the base-3 decode."""
    import torch
    m = Model(wl, layers, "cuda:0", base3=True)
    m.set_tokens(1)
    sec, _ = run_steps(m, steps, warmup, use_graph)
    weights = sum(M * K for M, K in wl.shapes) * layers
    res = {"ms_per_step": round(sec * 1e3, 4),
           "packed_gb": round(m.packed_bytes / 1e9, 3),
           "packed_gb_per_s": round(m.packed_bytes / sec / 1e9, 1),
           "frac_of_hbm_peak": round(m.packed_bytes / sec / 1e9 / PEAK_HBM_GBS, 4),
           "t_weights_per_s": round(weights / sec / 1e12, 2),
           "t_weights_per_s_2bit": round(weights / sec_2bit / 1e12, 2),
           "step_speedup_over_2bit": round(sec_2bit / sec, 3)}
    del m
    torch.cuda.empty_cache()
    return res


def small_configs_extra(steps, warmup, use_graph):
    """The single 2560 x 2560 GEMV and the 2B-style block at 1 and 64 tokens,
    hot (the same weights every call: they stay in the 256 MB last-level
    cache) and cold (distinct weight copies in rotation, more than 256 MB in
    all), per call of the whole path (quantization included)."""
    import torch
    import ternary_weight_quantized_bt_amd as bt
    import workloads as W
    dev = "cuda:0"
    res = {}
    # single GEMV from the float token: bt_ternary_linear (one launch, the
    # token quantized in the kernel's prologue); beside it the two-call path
    # (bt_quant_act, then bt_ternary_gemv)
    wl = W.GEMV_2560
    M, K = wl.shapes[0]
    x = W.layer_inputs(wl, 0, 1, dev)[0]
    xq = torch.empty((1, K), dtype=torch.int8, device=dev)
    xsc = torch.empty(1, dtype=torch.float32, device=dev)
    xsm = torch.empty(1, dtype=torch.int32, device=dev)
    y = torch.empty((1, M), dtype=torch.float32, device=dev)
    assert bt.bt_linear_one_launch(1, M, K, bt.BT_F32) == 1
    row = {}
    for name, copies in (("hot", 1), ("cold", 192)):
        ps = [bt.pack(W.ternary_weights(M, K, wl.weight_dist, W.weight_seed(wl, c, 0), dev), 0.02)
              for c in range(copies)]

        def step():
            for pk in ps:
                bt.bt_ternary_linear(pk, M, K, x, bt.BT_F32, 1, y, bt.BT_F32, None, 0)

        def step_two_calls():
            for pk in ps:
                bt.bt_quant_act(x, bt.BT_F32, 1, K, xq, xsc, xsm)
                bt.bt_ternary_gemv(pk, M, K, xq, xsc, xsm, 1, y, bt.BT_F32)
        reps = 20 if copies == 1 else 1
        sec, _ = run_steps(None, steps * reps, warmup * reps, use_graph, step=step,
                           per_graph=reps)
        sec2, _ = run_steps(None, steps * reps, warmup * reps, use_graph, step=step_two_calls,
                            per_graph=reps)
        per = sec / copies
        row[name] = {"copies": copies, "us_per_call": round(per * 1e6, 3),
                     "packed_gb_per_s": round(M * K / 4 / per / 1e9, 1),
                     "two_calls_us_per_call": round(sec2 / copies * 1e6, 3)}
        del ps
    res["gemv_2560"] = row
    for wl, N in ((W.LAYER2B_N1, 1), (W.LAYER2B_N64, 64)):
        row = {}
        for name, layers in (("hot", 1), ("cold", 16)):
            m = Model(wl, layers, dev)
            m.set_tokens(N)
            reps = 20 if layers == 1 else 1
            sec, _ = run_steps(m, steps * reps, warmup * reps, use_graph, per_graph=reps)
            per = sec / layers
            row[name] = {"blocks": layers, "us_per_block": round(per * 1e6, 3),
                         "packed_gb_per_s": round(wl.packed_bytes_per_layer / per / 1e9, 1),
                         "frac_of_hbm_peak": round(wl.packed_bytes_per_layer / per / 1e9 / PEAK_HBM_GBS, 4)}
            if N > 1:
                ops = 2 * N * sum(M * K for M, K in wl.shapes)
                row[name]["int8_tops"] = round(ops / per / 1e12, 1)
            del m
            torch.cuda.empty_cache()
        res[wl.name] = row
    return res


def copy_bandwidth_extra():
    """Device-to-device copies (torch), 1 MB to 8 GB: bytes read + written per
    second, the measured reference beside the 8 TB/s specification."""
    import torch
    res = {}
    for size in (1 << 20, 16 << 20, 256 << 20, 1 << 30, 4 << 30, 8 << 30):
        src = torch.ones(size, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        reps = max(3, min(200, (8 << 30) // size))
        for _ in range(3):
            dst.copy_(src)
        t, _ = time_region(lambda: dst.copy_(src), reps)
        res[f"{size >> 20}MB"] = round(2 * size * reps / t / 1e9, 1)
        del src, dst
        torch.cuda.empty_cache()
    return res


def base3_extra(steps, warmup, use_graph, layers=8):
    """The 70B-class block's seven matrices in both weight formats, one
    decode launch per matrix on activations quantized beforehand, `layers`
    blocks deep so that the weights stream from HBM rather than from the
    last-level cache: the 2-bit T16Q256 kernel against the base-3 B3T1024
    one (1.625 bits per weight), at 1 and 4 tokens."""
    import torch
    import ternary_weight_quantized_bt_amd as bt
    import workloads as W
    dev = "cuda:0"
    shapes = W.STREAM70B.shapes
    mats = []
    for l in range(layers):
        for i, (M, K) in enumerate(shapes):
            w = W.ternary_weights(M, K, "p0_0.4", 7000 + 10 * l + i, device=dev)
            mats.append((M, K, bt.pack(w, 0.02), bt.pack_b3(w, 0.02)))
            del w
    weights = layers * sum(M * K for M, K in shapes)
    fmt_bytes = {"t16q256_2bit": sum(m[2].numel() for m in mats),
                 "b3t1024_base3": sum(m[3].numel() for m in mats)}
    res = {"layers": layers, "launches_per_step": len(mats),
           "packed_gb": {k: round(v / 1e9, 3) for k, v in fmt_bytes.items()}}
    for N in (1, 4):
        acts = {K: bt.quant_act(W.activations(N, K, "normal", K + N, "bf16", device=dev))
                for K in sorted({K for _, K in shapes})}
        outs = {M: torch.empty((N, M), dtype=torch.bfloat16, device=dev)
                for M in sorted({M for M, _ in shapes})}
        row = {}
        for name, which, fn in (("t16q256_2bit", 2, bt.bt_ternary_gemv),
                                ("b3t1024_base3", 3, bt.bt_ternary_gemv_b3)):
            def step():
                for m in mats:
                    M, K = m[0], m[1]
                    xq, xsc, xsm = acts[K]
                    fn(m[which], M, K, xq, xsc, xsm, N, outs[M], bt.BT_BF16)
            sec, _ = run_steps(None, steps, warmup, use_graph, step=step)
            row[name] = {"ms_per_step": round(sec * 1e3, 4),
                         "packed_gb_per_s": round(fmt_bytes[name] / sec / 1e9, 1),
                         "frac_of_hbm_peak": round(fmt_bytes[name] / sec / 1e9 / PEAK_HBM_GBS, 4),
                         "t_weights_per_s": round(weights / sec / 1e12, 2)}
        row["base3_over_2bit_weights_per_s"] = round(
            row["b3t1024_base3"]["t_weights_per_s"] / row["t16q256_2bit"]["t_weights_per_s"], 3)
        res[f"{N}_token" + ("s" if N > 1 else "")] = row
    del mats
    torch.cuda.empty_cache()
    # Steady state: one tall matrix per launch (229376 x 8192, 1.9 G weights),
    # so that launch and prologue costs are amortized.
    M, K = 229376, 8192
    w = W.ternary_weights(M, K, "p0_0.4", 7777, device=dev)
    tall = {"t16q256_2bit": (bt.pack(w, 0.02), bt.bt_ternary_gemv),
            "b3t1024_base3": (bt.pack_b3(w, 0.02), bt.bt_ternary_gemv_b3)}
    del w
    xq, xsc, xsm = bt.quant_act(W.activations(1, K, "normal", 5, "bf16", device=dev))
    y = torch.empty((1, M), dtype=torch.bfloat16, device=dev)
    row = {"shape": [M, K], "tokens": 1}
    for name, (p, fn) in tall.items():
        def step():
            fn(p, M, K, xq, xsc, xsm, 1, y, bt.BT_BF16)
        sec, _ = run_steps(None, steps, warmup, use_graph, step=step)
        row[name] = {"us_per_launch": round(sec * 1e6, 2),
                     "packed_gb_per_s": round(p.numel() / sec / 1e9, 1),
                     "frac_of_hbm_peak": round(p.numel() / sec / 1e9 / PEAK_HBM_GBS, 4),
                     "t_weights_per_s": round(M * K / sec / 1e12, 2)}
    row["base3_over_2bit_weights_per_s"] = round(
        row["b3t1024_base3"]["t_weights_per_s"] / row["t16q256_2bit"]["t_weights_per_s"], 3)
    res["steady_state_tall_matrix"] = row
    del tall
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary)
        return
    if args.trace_summary:
        import workloads as W
        trace_summary(args.trace_summary, args.steps, args.warmup,
                      args.layers or W.BY_NAME[args.workload].layers)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); "
              "the library has no multi-GPU path", file=sys.stderr)
        sys.exit(2)
    import torch
    import workloads as W
    import ternary_weight_quantized_bt_amd as bt
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    bt.lib()  # fail loudly if the HIP library is missing

    if args.base3_only:
        res = base3_extra(args.steps, args.warmup, not args.no_graph, args.layers or 8)
        print(json.dumps({"base3_vs_2bit_70b": res}), flush=True)
        return

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": 1 << 30, "copies": 5}))
        return

    wl = W.BY_NAME[args.workload]
    layers = args.layers or wl.layers
    N = args.tokens or wl.batches[0]
    use_graph = not args.no_graph
    decode = N < bt.BT_PREFILL_MIN_N

    model = Model(wl, layers, "cuda:0")
    model.set_tokens(N)
    print(f"[bench] {wl.name}: {layers} layer(s), {N} token(s), "
          f"{model.packed_bytes / 1e9:.3f} GB packed, setup {model.setup_s:.1f} s",
          file=sys.stderr, flush=True)

    sec, wall = run_steps(model, args.steps, args.warmup, use_graph)
    note(f"timed steps done: {sec * 1e3:.4f} ms per step")
    eager_sec = None
    if use_graph:
        eager_sec, _ = run_steps(model, max(3, args.steps // 4), 2, False)
    # Grouped products alone, on inputs quantized beforehand (same kernels and
    # grids as the per-group step, minus the quantization).
    kt, launches = kernel_pass(model, max(3, args.steps // 2))
    ops_step = 2 * N * sum(M * K for M, K in wl.shapes) * layers
    fused = N <= 4 and all(n * k <= 65536 for k in wl.input_widths()
                           for n in [1 if N == 1 else (2 if N == 2 else 4)])
    if decode:
        value = model.packed_bytes / sec / 1e9
        unit = "GB/s"
        if model.one_launch:
            # One launch per layer and nothing else in the step: the kernel's
            # average duration is the step time over the layer count (HIP
            # events around the timed region, on the stream the graph runs on).
            kernel_name = "layer_dot4_kernel"
            launches_per_step = layers
            kavg = sec / launches_per_step
        elif fused:
            # Four launches per layer with the quantization fused into them:
            # again nothing else in the step.
            kernel_name = "decode_dot4_kernel (fused quantization)"
            launches_per_step = 4 * layers
            kavg = sec / launches_per_step
        else:
            kernel_name = "decode_dot4_kernel" if N <= 4 else "decode_mfma_kernel"
            launches_per_step = 4 * layers
            kavg = kt
        bytes_per_launch = model.packed_bytes / launches_per_step
        achieved = bytes_per_launch / kavg / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4)}
    else:
        kernel_name = "prefill_kernel"
        launches_per_step = 4 * layers
        bytes_per_launch = model.packed_bytes / launches_per_step
        kavg = kt
        value = ops_step / sec / 1e12
        unit = "TOPS"
        achieved = ops_step / launches_per_step / kavg / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_INT8_TOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / PEAK_INT8_TOPS, 4)}
    roofline["traffic"] = read_traffic(kernel_name, kernel_sha(kernel_name))
    roofline["kernel"] = kernel_name
    roofline["kernel_avg_us"] = round(kavg * 1e6, 3)
    # The same kernel's mean duration in a rocprofv3 kernel trace of this
    # command (timed dispatches only), while its sources are unchanged: it
    # excludes the gaps between launches that the event figure includes.
    tr = read_trace(kernel_name, kernel_sha(kernel_name)) if decode else None
    if tr:
        roofline["rocprof_kernel_avg_us"] = tr["mean_us"]
        roofline["rocprof_frac"] = round(bytes_per_launch / (tr["mean_us"] * 1e-6) / 1e9
                                         / PEAK_HBM_GBS, 4)
    roofline["launches_per_step"] = launches_per_step
    roofline["algorithmic_bytes_per_launch"] = int(bytes_per_launch)
    roofline["prequantized_group_kernel_avg_us"] = round(kt * 1e6, 3)

    extra = {}
    if not args.no_extra and decode and model.one_launch:
        spg, _ = run_steps(model, args.steps, args.warmup, use_graph, model.step_per_group)
        extra["same_step_per_group_launches"] = {
            "ms_per_step": round(spg * 1e3, 4),
            "packed_gb_per_s": round(model.packed_bytes / spg / 1e9, 2),
            "frac_of_hbm_peak": round(model.packed_bytes / spg / 1e9 / PEAK_HBM_GBS, 4),
        }
    if not args.no_extra and wl.name == "stream70b" and N == 1:
        model.set_tokens(8)
        s8, _ = run_steps(model, args.steps, args.warmup, use_graph)
        k8, _ = kernel_pass(model, max(3, args.steps // 2))
        extra["stream70b_8_tokens"] = {
            "ms_per_step": round(s8 * 1e3, 4),
            "packed_gb_per_s": round(model.packed_bytes / s8 / 1e9, 2),
            "frac_of_hbm_peak": round(model.packed_bytes / s8 / 1e9 / PEAK_HBM_GBS, 4),
            # one group's product launch on pre-quantized inputs, averaged
            # over the four groups (the step runs the four as one launch)
            "per_group_launch_avg_us": round(k8 * 1e6, 3),
            "int8_tops": round(16 * sum(M * K for M, K in wl.shapes) * layers / s8 / 1e12, 2),
        }
        tr8 = read_trace("decode_mfma_multi_kernel", kernel_sha("decode_mfma_multi_kernel"))
        if tr8:
            e8 = extra["stream70b_8_tokens"]
            e8["rocprof_product_kernel_us"] = tr8["mean_us"]
            e8["rocprof_product_frac_of_hbm_peak"] = round(
                _block_packed_bytes() / (tr8["mean_us"] * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)
            for k in ("quant_mean_us", "quant_to_product_gap_mean_us",
                      "quant_to_product_gap_median_us"):
                if k in tr8:
                    e8["rocprof_" + k] = tr8[k]
    packed_bytes_step = model.packed_bytes
    pack = {"seconds": round(model.pack_s, 3),
            "int8_weights_gb_per_s": round(4 * packed_bytes_step / model.pack_s / 1e9, 2)}
    if not args.no_extra:
        del model
        torch.cuda.empty_cache()
        note("extra: 2048-token prefill")
        extra["prefill2b_n2048"] = prefill_extra(args.steps, args.warmup, use_graph)
        note("extra: weight quantizer")
        extra["weight_quantizer_70b_gate"] = weight_quant_extra(args.steps, args.warmup)
        note("extra: base-3 against 2-bit matrices")
        extra["base3_vs_2bit_70b"] = base3_extra(args.steps, args.warmup, use_graph)
        if wl.name == "stream70b" and N == 1:
            note("extra: base-3 stream")
            extra["stream70b_1_token_base3"] = base3_stream_extra(wl, layers, args.steps,
                                                                  args.warmup, use_graph,
                                                                  value, sec)
        note("extra: small configurations")
        extra["small_configs_hot_and_cold"] = small_configs_extra(args.steps, args.warmup,
                                                                  use_graph)
        note("extra: device copies")
        copy = copy_bandwidth_extra()
        extra["device_copy_gb_per_s_read_plus_write"] = copy
        # copies of 1 GB and more run from HBM (smaller ones from the caches)
        hbm_copy = max(v for k, v in copy.items() if int(k[:-2]) >= 1024)
        extra["value_over_hbm_device_copy"] = round(value / hbm_copy, 4)

    cpu = None
    if not args.no_cpu:
        note("oracle on the host")
        cpu = cpu_baseline(wl, N, args.cpu_seconds)

    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(sec * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {
            "workload": wl.name, "description": wl.description, "tokens": N,
            "layers": layers, "projections_per_layer": len(wl.shapes),
            "packed_bytes_per_step": packed_bytes_step,
            "int8_ops_per_step": ops_step,
            "hip_graph": use_graph,
            "ms_per_step_eager": round(eager_sec * 1e3, 4) if eager_sec else None,
            "frac_of_hbm_peak" if decode else "frac_of_int8_peak":
                round(value / (PEAK_HBM_GBS if decode else PEAK_INT8_TOPS), 4),
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extra": extra,
        "pack_load_time": pack,
        "wall_s_timed_region": round(wall, 4),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
