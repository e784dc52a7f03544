"""GPU check of bench.py's roofline object on an MFMA-bound workload: Long
verify (four drafts per query, 725 FLOP per KV byte, above the 312.5 FLOP/B
spec ridge) must be reported against the matrix-core peaks, with the memory
view kept beside it."""

import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("form", ["one-launch", "per-rank"])
def test_long_verify_roofline_is_mfma_bound(form):
    cmd = [sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--workload", "long", "--steps", "1",
           "--warmup", "1", "--no-cpu-baseline", "--no-probe", "--no-secondary", "--power-seconds", "0"]
    if form == "one-launch":
        cmd.append("--one-launch")
    print("bench:", " ".join(cmd[2:]), flush=True)
    r = subprocess.run(cmd, cwd=ROOT, capture_output=True, text=True, timeout=110)
    assert r.returncode == 0, r.stderr[-2000:]
    line = json.loads(r.stdout.strip().splitlines()[-1])
    roof = line["roofline"]
    assert roof["bound"] == "mfma" and roof["unit"] == "TFLOP/s" and roof["peak"] == 2500.0
    # one launch's matrix rate: below the spec, above what the whole step averages
    assert 0.2 < roof["frac"] < 1.0
    assert roof["achieved"] >= line["tflops"] * 0.95
    # the launch's share of the step's FLOPs (2176 FLOP per visible token and
    # head): all of them for one launch of all stripes, one rank's eighth per call
    share = 1 if form == "one-launch" else 8
    assert roof["flops_per_launch"] * share == pytest.approx(line["tflops"] * 1e12 * line["ms_per_step"] * 1e-3,
                                                              rel=2e-3)
    hbm = roof["hbm_view"]
    assert hbm["unit"] == "GB/s" and 0.0 < hbm["frac"] < 1.0
