"""bench.py's host side on a machine without a GPU: the single-GPU contract
(a request for more GPUs is refused with a message, before any GPU work) and
the counter-traffic lookup (the committed summary is used only for the
kernel source it was taken on)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "single GPU" in r.stdout + r.stderr
    assert not any(line.startswith("{") for line in r.stdout.splitlines())


def test_counter_traffic_follows_the_kernel_source(tmp_path, monkeypatch):
    sha = bench.kernel_source_hash()
    (tmp_path / "profiles").mkdir()
    data = {"qwen2.5-72b-mlp/interleaved/config40": {
        "hbm_bytes_per_launch": 6479065631, "algorithmic_bytes": 1278214144,
        "kernel_source_sha": sha},
            "qwen2.5-1.5b-mlp/interleaved/config40": {
        "hbm_bytes_per_launch": 235100000, "algorithmic_bytes": 98041856,
        "kernel_source_sha": "0" * 16}}
    (tmp_path / "profiles" / "traffic.json").write_text(json.dumps(data))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.counter_traffic("qwen2.5-72b-mlp", 1, {"id": 40}) == 6479065631
    # a summary taken on another kernel source gives no traffic figure
    assert bench.counter_traffic("qwen2.5-1.5b-mlp", 1, {"id": 40}) is None
    # nor does another layout or configuration
    assert bench.counter_traffic("qwen2.5-72b-mlp", 0, {"id": 40}) is None
    assert bench.counter_traffic("qwen2.5-72b-mlp", 1, {"id": 41}) is None
    # nor a missing or unreadable file
    (tmp_path / "profiles" / "traffic.json").write_text("{not json")
    assert bench.counter_traffic("qwen2.5-72b-mlp", 1, {"id": 40}) is None


def test_committed_traffic_summaries_are_well_formed():
    data = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    assert data
    for key, v in data.items():
        assert v["hbm_bytes_per_launch"] > 0 and v["algorithmic_bytes"] > 0, key
        assert len(v["kernel_source_sha"]) == 16, key
