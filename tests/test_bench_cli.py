"""bench.py's contract on the CPU: one JSON line per run is produced only on
a GPU, but the refusal of several GPUs, the algorithmic byte counts the
roofline divides by, the rocprofv3 summary it formats and the validity of
the committed HBM counter figure can be checked here."""
import csv
import importlib.util
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_algorithmic_bytes_per_stream_layer_step():
    b = bench()
    # W = 375, re-base chunk 25: K+V window 384,000 + q/out 8,192 + new rows in
    # 1,024 + appended 1,024 + re-based K 374 x 512 / 25 = 7,659.52
    assert b.bytes_per_sl_step(b.CONFIGS[2]) == pytest.approx(401899.52)
    # compensated re-base every step: adds the residual read + write and its row
    assert b.bytes_per_sl_step(b.CONFIGS[1]) == pytest.approx(
        375 * 1024 + 8192 + 2048 + 374 * 512 + 2 * 374 * 512 + 512)
    # encoder: 750 cached frames of K+V, q/out, new rows in, appended rows (20 x 64)
    assert b.bytes_per_sl_step(b.CONFIGS[5]) == pytest.approx(3901440)
    # mixed windows: the 86/85/85 average of the three windows' figures
    per = {W: W * 1024 + 8192 + 2048 + (W - 1) * 512 / 25 for W in (375, 250, 188)}
    want = (86 * per[375] + 85 * per[250] + 85 * per[188]) / 256
    assert b.bytes_per_sl_step(b.CONFIGS[3]) == pytest.approx(want)


def test_committed_hbm_counters_are_reported_only_for_their_kernel_sources():
    """roofline.traffic is reported only while the kernel sources equal those
    the counters were taken from (null otherwise), and a reported figure is
    the committed one."""
    b = bench()
    data = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    assert data, "no committed counter figures"
    for key, ent in data.items():
        kernel, workload = key.rsplit("@", 1)
        got = b.load_traffic(kernel, workload)
        files = tuple(ent.get("kernel_src_files", b.ATTN_SOURCES))
        if ent["kernel_src_digest"] == b.kernel_source_digest(files):
            assert got == ent["hbm_bytes_per_launch"], key
        else:
            assert got is None, key
        assert ent["hbm_bytes_per_launch"] == pytest.approx(
            ent["fetch_kib_per_launch"] * 1024 * ent["fetch_scale"]
            + ent["write_kib_per_launch"] * 1024 * ent["write_scale"], rel=1e-6), key


def test_rocprof_summary_of_a_synthetic_trace(tmp_path):
    d = tmp_path / "run" / "host"
    d.mkdir(parents=True)
    with open(d / "t_kernel_trace.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for i, dur in enumerate([10_000, 12_000, 14_000]):
            w.writerow({"Kernel_Name": "k_a", "Start_Timestamp": 100_000 * i,
                        "End_Timestamp": 100_000 * i + dur})
        w.writerow({"Kernel_Name": "k_b", "Start_Timestamp": 5, "End_Timestamp": 2_005})
    out = bench().summarize_rocprof(str(tmp_path / "run"), last=2)
    lines = [l for l in out.splitlines() if l.strip().endswith("k_a")]
    assert len(lines) == 1
    calls, mean, median, last = lines[0].split()[:4]
    assert (int(calls), float(mean), float(median), float(last)) == (3, 12.0, 12.0, 13.0)


def test_launch_bytes_charge_each_timed_launch_its_own_work():
    """launch_bytes (the bytes the roofline divides by) per launch: over any 25
    consecutive full-window steps every stream re-bases exactly once, so the
    mean equals the amortised per-step figure; a launch without a re-base and
    a re-base launch carry their own bytes."""
    import numpy as np
    b = bench()
    c = b.CONFIGS[2]
    L, S = c["L"], c["S"]
    win, org = np.full(S, 375, np.int32), np.zeros(S, np.int64)
    steps = list(range(400, 425))
    mean = b.launch_bytes(c, win, org, steps) / len(steps)
    assert mean == pytest.approx(b.bytes_per_sl_step(c) * L * S)
    # origin 0, W = 375, chunk 25: the base moves when the oldest retained
    # position reaches a multiple of 25, i.e. at steps 399, 424, ...
    plain = (375 * 1024 + 8192 + 2048) * L * S
    assert b.launch_bytes(c, win, org, [400]) == plain
    assert b.launch_bytes(c, win, org, [399]) == plain + 374 * 512 * L * S
    # mixed windows and start offsets: the same identity stream by stream
    c3 = b.CONFIGS[3]
    S3 = c3["S"]
    w3 = np.repeat(np.array(c3["W"], np.int32), [86, 85, 85])
    o3 = np.random.default_rng(1).integers(0, 5000, S3).astype(np.int64)
    m3 = b.launch_bytes(c3, w3, o3, list(range(500, 525))) / 25
    assert m3 == pytest.approx(b.bytes_per_sl_step(c3) * c3["L"] * S3)
    # compensated re-base every step (one stream, one layer): every launch re-bases
    c1 = b.CONFIGS[1]
    assert b.launch_bytes(c1, np.array([375]), np.array([0]), [700]) == \
        pytest.approx(b.bytes_per_sl_step(c1))
    # compaction: rows attended grow from W + 1 to the capacity between
    # compactions; over one period the mean is the page's average length
    c4 = b.CONFIGS[4]
    W, cap = c4["W"], c4["cap"]
    period = list(range(cap, cap + (cap - W)))
    m4 = b.launch_bytes(c4, np.full(16, W), np.zeros(16, np.int64), period) / len(period)
    want = ((W + 1 + cap) / 2 * 1024 + 8192 + 2048) * c4["L"] * c4["S"]
    assert m4 == pytest.approx(want)
