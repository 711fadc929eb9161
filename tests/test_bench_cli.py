"""Host-side checks of bench.py (no GPU): the single-GPU contract, the
profile summaries and the traffic figure's source guard."""

import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_stats_summary_from_kernel_trace(tmp_path):
    d = tmp_path / "trace"
    d.mkdir()
    (d / "run_kernel_stats.csv").write_text(
        '"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs","StdDev"\n'
        '"void bsa::attn_fwd_kernel<128, false, 0>(bsa::AttnArgs)",10,9800000,980000.0,90.0,970000,990000,1.0\n'
        '"void bsa::select_kernel<128, 16, 8>(float const*)",10,450000,45000.0,4.1,44000,46000,1.0\n')
    log = tmp_path / "bench.log"
    log.write_text(json.dumps({"stages_ms": {"attention": 0.99}, "roofline": {"achieved": 828.0}}) + "\n")
    stats = bench.rocprof_stats(str(d))
    assert stats[0][0] == "bsa::attn_fwd_kernel<128, false, 0>" and stats[0][1] == 10
    assert abs(stats[0][2] - 980.0) < 1e-9
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--rocprof-summary", "stats", str(d),
                        "--bench-log", str(log), "--command", "CMD"], capture_output=True, text=True, cwd=ROOT,
                       timeout=300)
    assert r.returncode == 0, r.stderr
    assert r.stdout.startswith("command: CMD")
    assert "average 980.0 us" in r.stdout and "ratio events / kernel 1.010" in r.stdout


def test_traffic_figure_follows_the_source(tmp_path, monkeypatch):
    # the committed counter summary counts only for the attention sources it
    # was taken from
    t = tmp_path / "attn_fwd_hunyuan720_traffic.txt"
    t.write_text("traffic_bytes_per_launch: 4.5e+09\nsource_sha256: " + bench.attn_sources_sha() + "\n")
    monkeypatch.setattr(bench, "traffic_file", lambda wl: str(tmp_path / f"attn_fwd_{wl}_traffic.txt"))
    assert bench.measured_traffic("hunyuan720") == 4.5e9
    assert bench.measured_traffic("wan480") is None
    t.write_text("traffic_bytes_per_launch: 4.5e+09\nsource_sha256: 0000\n")
    assert bench.measured_traffic("hunyuan720") is None


def test_headline_is_the_720p_layer():
    # the metric names ~90 % sparsity on the largest layer: the 118,800-token
    # 720p one is the default workload, the 480p layer comes second
    import argparse
    src = open(os.path.join(ROOT, "bench.py")).read()
    assert 'ap.add_argument("--config", default="hunyuan720"' in src
    assert 'ap.add_argument("--also", default="wan480"' in src
    from gen import WORKLOADS
    assert WORKLOADS["hunyuan720"].n_valid == 118800
