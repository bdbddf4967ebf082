"""CPU checks of bench.py's contract: it refuses more than one GPU, its CPU
baseline leg (the oracle on whole heads) reports the fields the JSON line
carries, and the traffic lookup is tied to the kernels' source hash."""
import os
import subprocess
import sys

import bench
from workloads import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_cpu_baseline_fields():
    cb = bench.cpu_baseline(WORKLOADS[5], 0.1)      # stops after the first head
    assert set(cb) == {"value", "unit", "cores", "kind", "sample"}
    assert cb["kind"] == "oracle" and cb["unit"] == "TFLOP/s"
    assert cb["value"] > 0 and cb["cores"] >= 1
    assert cb["sample"].startswith("1 of 16 (b,h) heads of bwd-causal-B1H16S4096d128")


def test_traffic_summary_is_tied_to_the_source_hash(tmp_path, monkeypatch):
    sha = bench.kernel_sources_sha256("fwd_kernel")
    assert sha == bench.kernel_sources_sha256("fwd_kernel") and len(sha) == 64
    assert sha != bench.kernel_sources_sha256("fwd8_kernel")
    (tmp_path / "profiles").mkdir()
    path = tmp_path / "profiles" / "traffic_fwd_kernel_some-workload.md"
    path.write_text(f"- hbm_bytes_per_launch: `123456`\n- source_sha256: `{sha}`\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_sources_sha256", lambda k: sha)
    assert bench.read_traffic("fwd_kernel", "some-workload") == 123456
    path.write_text(f"- hbm_bytes_per_launch: `123456`\n- source_sha256: `{'0' * 64}`\n")
    assert bench.read_traffic("fwd_kernel", "some-workload") is None
    assert bench.read_traffic("fwd_kernel", "no-such-workload") is None
