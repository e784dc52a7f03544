"""bench.py's contract that needs no GPU: it measures one GPU and says so."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "single MI355X" in r.stderr


def test_bench_help_lists_the_modes():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"], capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0
    for flag in ("--workload", "--op", "--multi", "--parts", "--topk", "--softcap", "--window", "--sinks",
                 "--streams", "--graph"):
        assert flag in r.stdout


def test_two_streams_with_one_launch_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--streams", "2", "--multi"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "--multi" in r.stderr


def test_graph_with_two_streams_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--graph", "--streams", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "--graph" in r.stderr
