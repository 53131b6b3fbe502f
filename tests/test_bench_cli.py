"""bench.py's command-line contract that holds without a GPU: a run on more than one GPU is
refused with a message (before anything touches a device), and the counter-traffic constants
are keyed to the kernel sources they were measured on (a changed source gives null, never a
stale figure)."""

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
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout.strip() == ""          # no JSON line for a run that did not happen


def test_traffic_constants_follow_their_sources(tmp_path, monkeypatch):
    for spec in (bench.ATTN_TRAFFIC, bench.ACCEPT_TRAFFIC):
        got = bench.traffic_bytes(spec)
        if got is not None:                # measured on these sources: a positive byte count
            assert got > 0
        # the same constants against a copy of the sources with one byte changed: null
        root = tmp_path / "copy"
        for f in spec["sources"]:
            dst = root / f
            dst.parent.mkdir(parents=True, exist_ok=True)
            dst.write_bytes(open(os.path.join(ROOT, f), "rb").read())
        first = root / spec["sources"][0]
        first.write_bytes(first.read_bytes() + b"\n")
        monkeypatch.setattr(bench, "ROOT", str(root))
        assert bench.traffic_bytes(spec) is None
        monkeypatch.setattr(bench, "ROOT", ROOT)
    json.dumps(bench.ATTN_TRAFFIC, default=str)
