"""bench.py's contract on the CPU: a multi-GPU request exits with a message
before touching a GPU, and measured HBM traffic is reported only while the
profiled kernel sources are unchanged."""

import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_traffic_is_reported_only_for_the_profiled_sources(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("kernel v1\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    rec = {"fwd_kernel<128>": {"sources": ["k.hip"], "source_sha256": bench.kernel_source_hash(["k.hip"]),
                               "fetch_bytes": 3.0e9, "write_bytes": 1.0e9}}
    traffic = tmp_path / "traffic.json"
    traffic.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC", str(traffic))
    assert bench.measured_traffic("fwd_kernel<128>") == 4.0e9
    assert bench.measured_traffic("merge_kernel<128>") is None
    src.write_text("kernel v2\n")  # the kernel changed after its counters were taken
    assert bench.measured_traffic("fwd_kernel<128>") is None


def test_committed_traffic_records_match_the_committed_kernel_sources():
    """profiles/traffic.json was taken on the kernels as they are: every
    record's source hash matches, so the bench line reports its traffic."""
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as fh:
        recs = json.load(fh)
    assert recs
    for kernel, rec in recs.items():
        assert rec["source_sha256"] == bench.kernel_source_hash(rec["sources"]), kernel
        assert bench.measured_traffic(kernel) == rec["fetch_bytes"] + rec["write_bytes"]
