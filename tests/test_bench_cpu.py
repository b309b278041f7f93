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
    data = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    sha = bench.kernel_source_hash()
    keys = [k for k, v in data.items() if "/" in k and v.get("kernel_source_sha") == sha]
    # the headline workload's table choice has a summary on the current source
    assert any(k.startswith("qwen2.5-72b-mlp/interleaved/") for k in keys), sorted(data)
    k = next(k for k in keys if k.startswith("qwen2.5-72b-mlp/interleaved/"))
    cfg = int(k.rsplit("config", 1)[1])
    got = bench.counter_traffic("qwen2.5-72b-mlp", 1, {"id": cfg})
    assert got == data[k]["hbm_bytes_per_launch"] and got > data[k]["algorithmic_bytes"]
    # another kernel source: no traffic figure
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 16)
    assert bench.counter_traffic("qwen2.5-72b-mlp", 1, {"id": cfg}) is None
    # an unknown configuration: none either
    monkeypatch.undo()
    assert bench.counter_traffic("qwen2.5-72b-mlp", 1, {"id": 9999}) is None
