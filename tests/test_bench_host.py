"""Host-side logic of bench.py (no GPU): the kernel-trace summary keeps the
per-layer kernel's dispatches of the timed steps only."""
import json

import bench


def _write_trace(folder, rows):
    folder.mkdir(parents=True, exist_ok=True)
    with open(folder / "run_kernel_trace.csv", "w") as f:
        f.write("Kind,Kernel_Name,Start_Timestamp,End_Timestamp\n")
        for name, b, e in rows:
            f.write(f'KERNEL_DISPATCH,"{name}",{b},{e}\n')


HEAD = "void bt::(anonymous namespace)::layer_dot4_kernel<unsigned short, 1, 16, 8, 3, false>(bt::LayerArgs)"
BASE3 = "void bt::(anonymous namespace)::layer_dot4_kernel<unsigned short, 1, 16, 4, 2, true>(bt::LayerArgs)"
FOUR = "void bt::(anonymous namespace)::layer_dot4_kernel<unsigned short, 4, 16, 8, 3, false>(bt::LayerArgs)"


def test_trace_summary_takes_the_timed_window(tmp_path):
    layers, warmup, steps = 3, 2, 4
    rows, t = [], 0
    # eager step + warm-up replays: 10 us each; timed replays: 20 us with
    # 1 us gaps; then later launches (eager timing) at 50 us, other kernels
    for i in range(layers * (1 + warmup)):
        rows.append((HEAD, t, t + 10_000))
        t += 12_000
        rows.append(("quant_onepass_kernel<>", t, t + 500))
        t += 1000
    t0 = t
    for i in range(layers * steps):
        rows.append((HEAD, t, t + 20_000))
        rows.append((BASE3 if i % 2 else FOUR, t + 5, t + 6))  # other instances, ignored
        t += 21_000
    for i in range(layers * 5):
        rows.append((HEAD, t, t + 50_000))
        t += 51_000
    _write_trace(tmp_path / "trace" / "host", rows[::-1])  # any order on disk
    out = tmp_path / "kernel_trace.json"
    e = bench.trace_summary(str(tmp_path / "trace"), steps, warmup, layers, out=str(out))
    assert e["timed_dispatches"] == layers * steps
    assert e["mean_us"] == e["median_us"] == e["min_us"] == e["max_us"] == 20.0
    span = layers * steps * 21_000 - 1_000
    assert e["window_span_ms"] == round(span / 1e6, 4)
    assert abs(e["busy_fraction_of_span"] - layers * steps * 20_000 / span) < 1e-4
    assert json.load(open(out))["layer_dot4_kernel"]["mean_us"] == 20.0
    assert t0 > 0
