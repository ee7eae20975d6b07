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


def test_committed_hbm_counters_match_the_kernel_sources():
    """The default line's roofline.traffic is reported only while the
    attention sources equal those the counters were taken from."""
    b = bench()
    data = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    ent = data["attn_kernel<128,4,decode_fused>@config2"]
    assert ent["kernel_src_digest"] == b.kernel_source_digest(), \
        "kernel sources changed since the counters in profiles/traffic.json were taken"
    assert b.load_traffic("attn_kernel<128,4,decode_fused>", "config2") == \
        ent["hbm_bytes_per_launch"]
    # the measured bytes agree with the algorithmic bytes of a launch within 1 %
    alg = b.bytes_per_sl_step(b.CONFIGS[2]) * 36 * 64
    assert abs(ent["hbm_bytes_per_launch"] / alg - 1) < 0.01


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
