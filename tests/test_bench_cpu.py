"""The benchmark's host-side contract (no GPU): the single-GPU guard, the
traffic lookup from a counter summary, and the CPU-baseline record."""
import json
import os
import subprocess
import sys
import types

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_lookup_follows_the_source_hash(tmp_path):
    src = tmp_path / "kernel.hip"
    src.write_text("// a kernel\n")
    rec = {"source_sha256": bench.source_sha256(str(src)), "hbm_bytes_per_launch": 1234}
    summary = tmp_path / "summary.md"
    summary.write_text("# counters\n\nTRAFFIC_JSON: " + json.dumps(rec) + "\n")
    assert bench.measured_traffic(str(summary), str(src)) == 1234
    src.write_text("// a kernel, changed\n")  # stale summary: no traffic figure
    assert bench.measured_traffic(str(summary), str(src)) is None
    assert bench.measured_traffic(str(tmp_path / "missing.md"), str(src)) is None


def test_traffic_hash_covers_the_included_headers(tmp_path):
    src, hdr = tmp_path / "kernel.hip", tmp_path / "common.h"
    src.write_text("#include \"common.h\"\n")
    hdr.write_text("// shared device code\n")
    files = [str(src), str(hdr)]
    rec = {"source_sha256": bench.source_sha256(files), "hbm_bytes_per_launch": 99}
    summary = tmp_path / "summary.md"
    summary.write_text("TRAFFIC_JSON: " + json.dumps(rec) + "\n")
    assert bench.measured_traffic(str(summary), files) == 99
    hdr.write_text("// shared device code, changed\n")  # a header edit makes the record stale
    assert bench.measured_traffic(str(summary), files) is None
    for lst in (bench.STREAM_SRC, bench.STREAM_Q_SRC, bench.TILE_SRC, bench.TILE_Q_SRC):
        assert all(os.path.exists(f) for f in lst)


def test_keyed_traffic_lines_pick_their_workload(tmp_path):
    src = tmp_path / "kernel.hip"
    src.write_text("// a kernel\n")
    h = bench.source_sha256(str(src))
    summary = tmp_path / "summary.md"
    summary.write_text("".join(
        f"TRAFFIC_JSON[{k}]: " + json.dumps({"source_sha256": h, "hbm_bytes_per_launch": v}) + "\n"
        for k, v in (("a", 10), ("b", 20))))
    assert bench.measured_traffic(str(summary), str(src), "b") == 20
    assert bench.measured_traffic(str(summary), str(src), "a") == 10
    assert bench.measured_traffic(str(summary), str(src), "c") is None
    assert bench.measured_traffic(str(summary), str(src)) is None  # no unkeyed line


def test_cpu_baseline_record():
    cfg = synth.CONFIGS["tiny_fp32"]
    wr, bias = synth.gen_router(cfg)
    wl = types.SimpleNamespace(cfg=cfg, x_host=synth.gen_x(cfg), wr_host=wr, bias_host=bias,
                               w_host=synth.gen_experts(cfg))
    rec = bench.cpu_baseline(wl, budget_s=0.2)
    assert rec["kind"] == "oracle" and rec["unit"] == "tokens/s"
    assert rec["value"] > 0 and rec["cores"] >= 1
    assert rec["value_1_thread"] is None or rec["value_1_thread"] > 0
    assert "tokens" in rec["sample"]
    assert set(rec["host"]) == {"cpu_model", "os_cpu_count", "OMP_NUM_THREADS"}
