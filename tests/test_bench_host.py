"""bench.py's host-side contract, on the CPU: one GPU only, and the attend
kernel's HBM traffic taken from the recorded counter runs only while the
kernel's sources are the ones the counters were taken on."""
import json
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    env = dict(os.environ, CUDA_VISIBLE_DEVICES="", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU only" in r.stderr and "--gpus 2" in r.stderr
    assert r.stdout.strip() == ""


def _records(qk):
    with open(bench.TRAFFIC_FILES[qk]) as f:
        return [json.loads(m.group(1)) for m in re.finditer(r"<!-- traffic (\{.*?\}) -->", f.read())]


@pytest.mark.parametrize("qk", ["bf16", "int8"])
def test_recorded_traffic_follows_the_kernel_digest(qk, tmp_path, monkeypatch):
    """Each record carries the fetch and write counts, their calibration
    factors and the bytes they give; the bench reports those bytes for a
    record whose digest is the current sources' and nothing otherwise."""
    recs = _records(qk)
    assert recs, "no traffic record"
    for rec in recs:
        assert rec["kernel"] == bench.KERNEL_NAMES[qk]
        want = rec["fetch_kib"] * 1024 * rec["fetch_factor"] + rec["write_kib"] * 1024 * rec["write_factor"]
        # the factors are stored to five decimals, the bytes from the unrounded ones
        assert abs(rec["bytes_per_launch"] - want) <= 1e-5 * want
        got = bench._recorded_traffic(rec["workload"], qk)
        if rec["kernel_sha256"] == bench._kernel_digest(qk):
            assert got == float(rec["bytes_per_launch"])
        else:
            assert got is None
    assert bench._recorded_traffic("no such workload", qk) is None
    # a record for another source digest is never reported
    stale = dict(recs[0], kernel_sha256="0" * 64)
    p = tmp_path / "traffic.md"
    p.write_text(f"<!-- traffic {json.dumps(stale)} -->\n")
    monkeypatch.setitem(bench.TRAFFIC_FILES, qk, str(p))
    assert bench._recorded_traffic(stale["workload"], qk) is None
