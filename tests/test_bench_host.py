"""bench.py host-side behaviour that needs no GPU: more than one GPU is
refused with a message, and the forward traffic figure is tied to the
current kernel sources."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_traffic_figure_matches_sources_or_is_null():
    import bench
    t = bench.fwd_traffic()
    text = open(bench.TRAFFIC_FILE).read()
    if bench.fwd_kernel_sha256() in text:
        assert t is not None and t > 0
    else:
        assert t is None
