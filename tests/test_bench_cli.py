"""CPU: the benchmark's command-line contract that needs no GPU.

bench.py measures one GPU; asked for more it must stop with a message and a
non-zero status before touching a device. Its host-side summaries of
rocprofv3 output (the per-layer split of a kernel trace, the HBM bytes from
counter passes) are checked on synthetic files."""
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


def test_summarize_pmc_scales_by_the_copy_kernel(tmp_path):
    """--summarize-pmc on synthetic counter files: each counter is scaled by
    what it reads for the copy kernel of known size (here FETCH_SIZE counts
    half the bytes, WRITE_SIZE all of them), averaged over dispatches."""
    import csv
    import json
    copy = 256 << 20

    def write(sub, counter, vals):
        d = tmp_path / sub / "host" / "1"
        d.mkdir(parents=True)
        with open(d / "run_counter_collection.csv", "w", newline="") as f:
            w = csv.writer(f)
            w.writerow(["Kernel_Name", "Counter_Name", "Counter_Value"])
            for name, v in vals:
                w.writerow([name, counter, v])

    kib = 1024
    write("fetch", "FETCH_SIZE", [
        ("splitkv::probe_copy_kernel(...)", copy / 2 / kib),
        ("void splitkv::partial_mfma_kernel<128, 7>", 1000.0),
        ("void splitkv::partial_mfma_kernel<128, 7>", 1002.0),
        ("void splitkv::combine_kernel<128>", 300.0)])
    write("write", "WRITE_SIZE", [
        ("splitkv::probe_copy_kernel(...)", copy / kib),
        ("void splitkv::partial_mfma_kernel<128, 7>", 50.0),
        ("void splitkv::combine_kernel<128>", 4.0)])
    meta = tmp_path / "kernels.json"
    meta.write_text("log line\n" + json.dumps({
        "nkv": 32768, "n_splits": 128, "kv_bytes_per_partial": 2_000_000,
        "record_bytes": 500_000, "partial_src_sha256_16": "abc"}) + "\n")
    out = tmp_path / "traffic.json"
    p = _run("--summarize-pmc", str(tmp_path / "fetch"), str(tmp_path / "write"),
             "--kernels-json", str(meta), "--write-traffic", str(out))
    assert p.returncode == 0, p.stderr
    res = json.loads(out.read_text())
    assert res["fetch_scale"] == 2.0 and res["write_scale"] == 1.0
    assert res["partial_fetch_bytes"] == 1001 * kib * 2
    assert res["partial_write_bytes"] == 50 * kib
    assert res["combine_fetch_bytes"] == 300 * kib * 2
    assert res["combine_write_bytes"] == 4 * kib
    assert res["hbm_bytes_per_launch"] == 1001 * kib * 2 + 50 * kib
    assert res["fetch_over_algorithmic"] == round(1001 * kib * 2 / 2_000_000, 4)
    assert res["combine_fetch_over_records"] == round(300 * kib * 2 / 500_000, 4)
    assert res["partial_src_sha256_16"] == "abc"
