"""CPU: the benchmark's command-line contract that needs no GPU.

bench.py measures one GPU; asked for more it must stop with a message and a
non-zero status before touching a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120, env=env)


def test_more_than_one_gpu_is_refused():
    p = _run("--gpus", "2")
    assert p.returncode == 2
    assert "one GPU" in p.stderr
    assert p.stdout.strip() == ""


def test_world_size_above_one_is_refused():
    env = dict(os.environ, WORLD_SIZE="4")
    p = _run(env=env)
    assert p.returncode == 2
    assert "one GPU" in p.stderr


def test_summarize_trace_splits_layers(tmp_path):
    """--summarize-trace on a synthetic kernel trace: two replays of 3 layers
    with known durations and gaps, other dispatches in between."""
    import csv
    import json
    rows, t = [], 1000
    rows.append(("copyBuffer", t, t + 500))
    t += 10_000
    for _ in range(2):
        for _ in range(3):
            rows.append(("void splitkv::partial_mfma_kernel<128, 7>", t, t + 13_000))
            t += 13_000 + 1_500
            rows.append(("void splitkv::combine_kernel<128>", t, t + 2_000))
            t += 2_000 + 1_000
        rows.append(("probe_copy_kernel", t, t + 50_000))
        t += 60_000
    sub = tmp_path / "host" / "123"
    sub.mkdir(parents=True)
    with open(sub / "run_kernel_trace.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        # the tracer's row order is not the dispatch order
        for r in reversed(rows):
            w.writerow(r)
    out = tmp_path / "split.json"
    p = _run("--summarize-trace", str(tmp_path), "--layers", "3",
             "--write-traffic", str(out))
    assert p.returncode == 0, p.stderr
    res = json.loads(out.read_text())
    assert res["replays"] == 2 and res["layers"] == 3
    assert res["partial_us"] == 13.0 and res["combine_us"] == 2.0
    assert res["gap_partial_to_combine_us"] == 1.5
    assert res["gap_combine_to_partial_us"] == 1.0
    assert res["layer_period_us"] == 17.5
