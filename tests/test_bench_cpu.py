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


def test_hbm_traffic_record_matches_the_kernel_sources():
    # the headline's measured HBM bytes are reported only while the kernel
    # sources are the ones the counters were taken on: a kernel change needs
    # a fresh pair of FETCH_SIZE / WRITE_SIZE passes and a new record
    sys.path.insert(0, ROOT)
    import bench
    bf16 = "o_r bf16, lse_r fp32"
    got = bench.measured_traffic("k3")             # the headline: a per-rank call with fp32 o_r
    assert got is not None, "profiles/stripe_attn_k3_hbm_bytes.md does not match the current kernel sources"
    assert 1.0e9 < got < 1.5e9                     # one K3 stripe call: 1.21 GB of KV plus partials
    got16 = bench.measured_traffic("k3", "per-rank", bf16)
    assert got16 is not None and got16 < got       # bf16 o_r writes half the output bytes
    one = bench.measured_traffic("k3", "one-launch", bf16)
    assert one is not None, "profiles/stripe_attn_k3_one_launch_hbm_bytes.md does not match the kernel sources"
    assert 9.6e9 < one < 9.9e9                     # all 8 stripes: 9.66 GB of KV, queries and bf16 outputs
    # a record covers the workload, step form and output type it was taken on only
    assert bench.measured_traffic("dsv3", "one-launch", bf16) is None
    assert bench.measured_traffic("k3", "one-launch", "fp32") is None


def test_k3_call_bytes_from_the_oracle_counts():
    # the roofline numerator: per rank, the rows the oracle's striping hands
    # that rank (every K3 request has 131072 tokens, 8 stripes), the queries
    # and the outputs; the K3 mean is the figure the traffic record compares to
    import numpy as np
    sys.path.insert(0, ROOT)
    import bench
    from oracle import layout as OL
    B, S, N, H = 64, 131072, 8, 96
    per_req = OL.local_counts(S, N, 1)                       # rows of one request on each rank
    local = np.tile(np.asarray(per_req, dtype=np.int64), (B, 1))
    got = bench.stripe_call_bytes(local, B, H)
    assert list(per_req) == [S // N] * N
    expect = B * (S // N) * 1152 + B * H * 1152 + B * H * 513 * 4
    assert (got == expect).all() and int(got.mean()) == 1227644928
    # four unmerged parts per request write four times the outputs
    assert (bench.stripe_call_bytes(local, B, H, 4) - got == 3 * B * H * 513 * 4).all()


def test_records_to_host_reorders_owner_order_to_request_order():
    # the records step leaves the merged result and every rank's records in
    # head-owner order [owner][B*q_len][H/N]; the parity leg reads them back in
    # request order [B][q_len][H]
    import types
    import numpy as np
    import torch
    sys.path.insert(0, ROOT)
    import bench
    w = types.SimpleNamespace(B=2, q_len=3, H=8)
    N, Hl = 4, 2
    g = torch.Generator().manual_seed(5)
    o_req = torch.randn((2, 3, 8, 512), generator=g)
    lse_req = torch.randn((2, 3, 8), generator=g)
    o_own = o_req.reshape(6, N, Hl, 512).permute(1, 0, 2, 3).contiguous()
    l_own = lse_req.reshape(6, N, Hl).permute(1, 0, 2).contiguous()
    recs = torch.zeros((N, N, 6, Hl, 516), dtype=torch.int16)
    for r in range(N):
        recs[r, ..., :512] = (o_own + r).to(torch.bfloat16).view(torch.int16)
        recs[r, ..., 512:514] = (l_own + r).unsqueeze(-1).contiguous().view(torch.int16)
    oh, lh, op, lp = bench.records_to_host(recs, o_own.reshape(-1, 512), l_own.reshape(-1), w)
    assert np.array_equal(oh, o_req.numpy()) and np.array_equal(lh, lse_req.numpy())
    for r in range(N):
        assert np.array_equal(lp[r], (lse_req + r).numpy())
        assert np.array_equal(op[r], (o_req + r).to(torch.bfloat16).float().numpy())


def test_power_sampler_parses_amd_smi(tmp_path, monkeypatch):
    # a stand-in amd-smi on PATH printing the layout of `amd-smi list` and of
    # `amd-smi metric --power --clock` (socket power, then one CLK line per XCD)
    sys.path.insert(0, ROOT)
    import bench
    xcds = "".join(f"        GFX_{i}:\n            CLK: {1500 + 10 * i} MHz\n            MIN_CLK: 500 MHz\n"
                   for i in range(8))
    metric = f"GPU: 0\n    POWER:\n        SOCKET_POWER: 1400 W\n    CLOCK:\n{xcds}        MEM_0:\n            CLK: 2000 MHz\n"
    (tmp_path / "metric.txt").write_text(metric)
    tool = tmp_path / "amd-smi"
    tool.write_text("#!/bin/sh\nif [ \"$1\" = list ]; then printf 'GPU: 0\\n    BDF: 0000:a4:00.0\\n'; "
                    f"else cat {tmp_path / 'metric.txt'}; fi\n")
    tool.chmod(0o755)
    monkeypatch.setenv("PATH", f"{tmp_path}:{os.environ['PATH']}")
    import time
    got = bench.sample_power(lambda: time.sleep(0.005), 1.5, sync=lambda: None)
    assert got["samples"] >= 1 and got["socket_w_mean"] == 1400.0 and got["xcds"] == 8
    assert got["gfx_mhz_mean"] == 1535.0 and got["gfx_mhz_min"] == 1535.0
    # two GPUs listed: the sampler cannot tell which is this process's
    tool.write_text("#!/bin/sh\nprintf 'GPU: 0\\nGPU: 1\\n'\n")
    assert "skipped" in bench.sample_power(lambda: None, 0.1, sync=lambda: None)
