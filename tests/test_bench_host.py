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


QUANT = "void bt::(anonymous namespace)::quant_onepass_kernel<unsigned short, 8, 128>(bt::QuantJobs)"
MULTI = "void bt::(anonymous namespace)::prefill_multi_kernel<4, 4, 4, 1, 2>(bt::(anonymous namespace)::MultiArgs)"
SINGLE = "void bt::(anonymous namespace)::prefill_kernel<4, 4, 4, 1, 2>(bt::GroupArgs, long)"


def test_grouped_window_pairs_each_product_with_its_quantization():
    # 2 skipped steps (quant 5 us, product 100 us), 3 timed steps (quant 7 us,
    # 2 us gap, product 110 us), then single-group launches that do not count
    rows, t = [], 0
    for i in range(5):
        timed = i >= 2
        q = 7_000 if timed else 5_000
        rows.append((QUANT, t, t + q))
        t += q + (2_000 if timed else 1_000)
        rows.append((MULTI, t, t + (110_000 if timed else 100_000)))
        t += 120_000
    for i in range(4):
        rows.append((SINGLE, t, t + 30_000))
        t += 31_000
    g = bench._grouped_window(rows, "prefill_multi_kernel<", 2, 3)
    assert g["timed_dispatches"] == 3 and g["skipped_dispatches"] == 2
    assert g["mean_us"] == g["min_us"] == 110.0
    assert g["quant_mean_us"] == 7.0
    assert g["quant_to_product_gap_mean_us"] == 2.0
    assert g["quant_to_product_gap_median_us"] == 2.0
    assert bench._grouped_window(rows, "prefill_multi_kernel<", 3, 3) is None


def test_prefill_step_counts():
    assert bench.prefill_steps(20, 50) == (200, 2000)
    assert bench.prefill_steps(450, 2010) == (440, 2000)
