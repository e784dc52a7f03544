"""Decode-step benchmark of DCP stripe attention + LSE merge on one MI355X.

One step = the N per-rank dcp_stripe_attn calls, each at its real per-rank
shape (all H query heads against that rank's stripe of every request) with
its chunk combine, plus one dcp_lse_merge of the N partials, all on one
stream with the inputs already resident in HBM.  Default workload: the
Kimi-K3-shaped decode batch (B=64 requests x 131072 tokens, H=96, N=8
stripes, page 64, base-2 LSE).

Prints one JSON line: KV GB/s as `value`, microseconds per step, the roofline
of the dominant launch (timed with HIP events on its stream), the float64 CPU
oracle timed on a bounded sample of the same workload on this host's cores
with the parity of the step's outputs against it, and the same step with the
N stripe attentions in one dcp_stripe_attn_multi launch (on one GPU the
ranks' attentions are independent work), timed beside it.

Other modes (not the headline): --one-launch times that form as the step
(the per-rank form beside it); --o-bf16 writes o_r in bf16 (the float32
result rounded once, lse_r float32: the partial payload the pages size at
(512 + 4) x 2 bytes per (row, head)) and merges with dcp_lse_merge_bf16;
--softcap / --window / --sinks time the step with a mergeable variant
switched on; --op relayout / head-return / stream / mfma time the relayout,
the head-return exchange and the two probes behind the measured peaks.
"""

from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
ROW_BYTES = 576 * 2             # one latent row (key = whole row, value = first 512 dims)
FLOP_PER_ROW_QUERY = 2 * 576 + 2 * 512   # QK^T + PV per (query row, visible token)


class FenceFreeEvent:
    """A HIP timing event created with hipEventDisableSystemFence: its record
    writes the timestamp without the system-scope release (L2 write-back and
    invalidation) a default event performs, which the HIP documentation names
    for events used only to measure time.  Between two kernels of one stream a
    default event's fence costs GPU time of its own (several microseconds);
    the steps here are read only after a device-wide synchronize, which orders
    everything.  Same record / elapsed_time interface as torch.cuda.Event."""
    _hip = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    @classmethod
    def hip(cls):
        if cls._hip is None:
            h = ctypes.CDLL("libamdhip64.so")
            h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            h.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._hip = h
        return cls._hip

    def __init__(self):
        self.ev = ctypes.c_void_p()
        rc = self.hip().hipEventCreateWithFlags(ctypes.byref(self.ev), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")

    def record(self, stream):
        rc = self.hip().hipEventRecord(self.ev, ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_time(self, other) -> float:
        ms = ctypes.c_float(0.0)
        rc = self.hip().hipEventElapsedTime(ctypes.byref(ms), self.ev, other.ev)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)

    def __del__(self):
        if self.ev and FenceFreeEvent._hip is not None:
            FenceFreeEvent._hip.hipEventDestroy(self.ev)
            self.ev = ctypes.c_void_p()


EVENT_KIND = "nofence"


def timing_event():
    """An event for the timed steps: fence-free (default) or torch's default one."""
    if EVENT_KIND == "torch":
        import torch
        return torch.cuda.Event(enable_timing=True)
    return FenceFreeEvent()


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: 20 for k3 and long, 100 for the short workloads)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed steps first (default: 10, or 20)")
    ap.add_argument("--workload", default="k3", help="tiny | dsv3 | k3 | ragged | long")
    ap.add_argument("--interleave", type=int, default=1)
    ap.add_argument("--splits", type=int, default=0, help="KV splits per request (0 = library's choice)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-unsharded-baseline", action="store_true",
                    help="time only the oracle's striped attention + merge, not also its unsharded attention")
    ap.add_argument("--op", default="step", choices=["step", "relayout", "head-return", "stream", "mfma"],
                    help="step: stripe attention + merge (the headline); relayout: prefill-to-decode relayout; "
                         "head-return: pack by head owner + the owners' merges; stream: the streaming-read probe "
                         "(measured HBM read peak) in every load mode; mfma: the MFMA probe (measured bf16 matrix "
                         "peak with the stripe kernel's 32x32x16 instruction)")
    ap.add_argument("--no-probe", action="store_true",
                    help="step: skip the streaming-read probe that gives the measured HBM peak")
    ap.add_argument("--softcap", type=float, default=0.0, help="logit softcap of the step (0 = none)")
    ap.add_argument("--window", type=int, default=0, help="sliding window of the step (0 = none)")
    ap.add_argument("--sinks", action="store_true", help="per-head attention sinks (on the last rank)")
    ap.add_argument("--flush-mib", type=int, default=-1,
                    help="MiB of scratch written between timed steps so the KV is not served from the memory-side "
                         "cache (-1: 1024 when the workload's KV is under 1 GiB, else 0); with a flush the step time "
                         "is the mean of the HIP-event step times")
    ap.add_argument("--one-launch", "--multi", dest="multi", action="store_true",
                    help="time the one-launch form as the step: the N stripe attentions as one "
                         "dcp_stripe_attn_multi launch (then the merge); the default step is the per-rank form, N "
                         "dcp_stripe_attn calls (the launch one rank runs on its own GPU) then the merge, and the "
                         "one-launch form is timed beside it")
    ap.add_argument("--topk", type=int, default=0,
                    help="k > 0: sparse attention over a global top-k selection per query token (plan + attention "
                         "on every rank)")
    ap.add_argument("--parts", type=int, default=0,
                    help="k > 0: every rank writes k unmerged parts per request and one merge folds all N*k")
    ap.add_argument("--records", action="store_true",
                    help="every rank writes its (o_r, lse_r) as bf16 records (+ fp32 lse) in head-owner order -- "
                         "the head-return all-to-all send buffer -- and one dcp_merge_heads over all owners' rows "
                         "folds the N ranks' records")
    ap.add_argument("--o-bf16", action="store_true",
                    help="every rank writes o_r in bf16 (the float32 result rounded once; lse_r stays float32), the "
                         "partial payload of page 'MLA 的 DCP' section 5, and dcp_lse_merge_bf16 merges them; by "
                         "default o_r is float32 and dcp_lse_merge merges them")
    ap.add_argument("--streams", type=int, default=1, choices=[1, 2],
                    help="2: the per-rank calls alternate between two streams, each with its own workspace, so "
                         "one rank's launch starts on the compute units the previous one leaves idle at its end "
                         "(the step time then has no per-launch split)")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step (every call of it) in a HIP graph and time its replays (the step time "
                         "then has no per-launch split)")
    ap.add_argument("--cpu-sample-requests", type=int, default=64,
                    help="requests of the workload the CPU oracle is timed on (bounded sample)")
    ap.add_argument("--events", default="nofence", choices=["nofence", "torch"],
                    help="timing events inside the timed steps: nofence (hipEventDisableSystemFence, the default) or "
                         "torch's default events, whose record also writes back and invalidates the caches")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the secondary measurement: the same step with all N stripes in one "
                         "dcp_stripe_attn_multi launch")
    ap.add_argument("--power-seconds", type=float, default=4.0,
                    help="after the timed region, loop the step this long while amd-smi samples socket power and "
                         "GFX clocks (0: off); reported as `power` in the JSON line")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after the timed region, run one plain device copy of this many MiB (the reference "
                         "kernel for scaling HBM byte counters)")
    args = ap.parse_args()
    # timing protocol: 20 timed steps for the long-running shapes, 100 for the
    # short ones (whose step is a few hundred microseconds)
    if args.streams > 1 and args.multi:
        print("--streams 2 splits the per-rank calls over two streams; --multi makes one launch", file=sys.stderr)
        sys.exit(2)
    if args.topk > 0 and args.multi:
        print("--topk plans and times each rank's selection with its call: per-rank form only", file=sys.stderr)
        sys.exit(2)
    if args.records and args.o_bf16:
        print("--records already writes bf16 outputs; --o-bf16 is the plain-layout form", file=sys.stderr)
        sys.exit(2)
    short = args.op == "step" and args.workload not in ("k3", "long")
    if args.steps is None:
        args.steps = 100 if short else 20
    if args.warmup is None:
        args.warmup = 20 if short else 10
    return args


# counter records of HBM traffic: one per step form (the per-rank call, the one launch of all stripes)
TRAFFIC_RECORDS = [os.path.join(ROOT, "profiles", "stripe_attn_k3_hbm_bytes.md"),
                   os.path.join(ROOT, "profiles", "stripe_attn_k3_one_launch_hbm_bytes.md")]


def stripe_call_bytes(local_rows, B: int, M: int, parts: int = 1, out_row_bytes: int = (512 + 1) * 4):
    """Algorithmic bytes of each rank's dcp_stripe_attn call: its latent rows
    (local_rows [B, N]: rows of request b on rank r, each read once), the
    queries (B x M rows of 576 bf16) and its outputs (o_r fp32 x 512 and lse_r,
    or `parts` unmerged parts of them; out_row_bytes per (row, head): 2052, or
    1032 for a bf16 record).  Returns one value per rank."""
    local_rows = np.asarray(local_rows, dtype=np.int64)
    q_bytes = B * M * ROW_BYTES
    out_bytes = parts * B * M * out_row_bytes
    return local_rows.sum(axis=0) * ROW_BYTES + q_bytes + out_bytes


def measured_traffic(workload: str, form: str = "per-rank", outputs: str = "fp32"):
    """HBM bytes of the dominant launch from a committed counter record: one
    dcp_stripe_attn call (form "per-rank": the attention kernel and its chunk
    combine) or one dcp_stripe_attn_multi launch of all stripes (form
    "one-launch"), with the given output type.  None when no record covers
    this workload, form and output type or the kernel sources changed since the
    counters were taken."""
    import hashlib
    for path in TRAFFIC_RECORDS:
        try:
            with open(path) as f:
                lines = [l.strip() for l in f if l.strip().startswith("traffic-record ")]
        except OSError:
            continue
        for line in lines:
            rec = json.loads(line[len("traffic-record "):])
            if rec.get("workload") != workload or rec.get("form") != form or rec.get("outputs") != outputs:
                continue
            h = hashlib.sha256()
            for src in rec["sources"]:
                with open(os.path.join(ROOT, src), "rb") as f:
                    h.update(f.read())
            return int(rec["bytes_per_call"]) if h.hexdigest() == rec["sha256"] else None
    return None


def main():
    global EVENT_KIND
    args = parse()
    EVENT_KIND = args.events
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU: the per-rank stripe kernels of all N stripes and the merge run on a "
              f"single MI355X; --gpus {args.gpus} (WORLD_SIZE={world}) is not supported.", file=sys.stderr)
        sys.exit(2)
    if args.records and args.parts:
        print("--records writes each rank's merged o_r as records; it does not take --parts", file=sys.stderr)
        sys.exit(2)
    if args.graph and args.streams > 1:
        print("--graph captures the one-stream step; it does not take --streams 2", file=sys.stderr)
        sys.exit(2)

    import torch
    from mla_context_kv_amd import dcp, stripes, workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.op == "relayout":
        run_relayout(args)
        return
    if args.op == "head-return":
        run_head_return(args)
        return
    if args.op == "stream":
        run_stream(args)
        return
    if args.op == "mfma":
        run_mfma(args)
        return
    dev = torch.device("cuda:0")
    w = workloads.WORKLOADS[args.workload]
    I = args.interleave
    N, P = w.N, w.page_size
    lay = dcp.layout(N, I, P)
    lens = workloads.seq_lens(w)
    base = 1 if w.lse_base == "2" else 0

    # ---- set-up (not timed): per-rank counts through the library, page tables,
    # inputs, owner-filtered write into the N pools
    t0 = time.perf_counter()
    counts = dcp.dcp_local_count(lay, torch.from_numpy(lens.astype(np.int64)).to(dev)).cpu().numpy()   # [B, N]
    tables, pool_pages = workloads.make_block_tables(w, stripes.pages_from_counts(counts, P))
    q = workloads.make_q(w, dev)
    kv = workloads.make_all_kv(w, lens, dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    sp = stripes.build_pools(lay, lens, kv, tables, pool_pages, status=status)
    ns = args.cpu_sample_requests
    sample = None
    if not args.no_cpu_baseline:
        # host copies (bf16) of the sampled requests' inputs; widened to float64
        # one request at a time, outside the oracle's timed calls
        off = 0
        sample = []
        for b in range(min(ns, w.B)):
            S = int(lens[b])
            sample.append((q[b].cpu(), kv[off:off + S].cpu(), S))
            off += S
    del kv
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    setup_s = time.perf_counter() - t0

    M = w.q_len * w.H
    K = max(args.parts, 1)                       # parts per rank (1: the rank's merged o_r)
    if args.records:
        # rank r's records: [owner d][B * q_len][H / N][516]; the merge output
        # is in the same owner order
        recs = torch.empty((N, N, w.B * w.q_len, w.H // N, 516), dtype=torch.int16, device=dev)
        o_parts = lse_parts = None
    else:
        o_parts = torch.empty((N * K, w.B, w.q_len, w.H, 512), dtype=torch.bfloat16 if args.o_bf16 else torch.float32,
                              device=dev)
        lse_parts = torch.empty((N * K, w.B, w.q_len, w.H), dtype=torch.float32, device=dev)
    o = torch.empty((w.B, w.q_len, w.H, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((w.B, w.q_len, w.H), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    # prebuilt argument blocks: the timed loop only calls into the library
    L = dcp.lib()
    attn_args = []
    ws_bytes = 0
    for r in range(N):
        a = dcp._attn_args(lay, r, q, sp.pools[r], sp.tables[r], sp.seq_len, workloads.SCALE, base,
                           args.parts if args.parts > 0 else args.splits, None, None, None, None,
                           partials=1 if args.parts > 0 else 0)
        a.out_records = 1 if args.records else 0
        a.o_bf16 = 1 if args.o_bf16 else 0
        need = ctypes.c_size_t(0)
        assert L.dcp_stripe_attn_workspace(ctypes.byref(a), ctypes.byref(need)) == 0
        ws_bytes = max(ws_bytes, need.value)
        attn_args.append(a)
    multi_arr = None
    if args.multi:
        multi_arr = (dcp.dcp_attn_args * N)(*attn_args)
        need = ctypes.c_size_t(0)
        assert L.dcp_stripe_attn_multi_workspace(multi_arr, N, ctypes.byref(need)) == 0
        ws_bytes = max(ws_bytes, need.value)
    workspaces = [torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev) for _ in range(args.streams)]
    streams = [stream] + [torch.cuda.Stream(dev) for _ in range(args.streams - 1)]   # default priority
    plans = None
    if args.topk > 0:
        # a global selection: k distinct visible positions per query token
        KT = args.topk
        topk = torch.full((w.B, w.q_len, KT), -1, dtype=torch.int32, device=dev)
        g = torch.Generator(device=dev).manual_seed(17)
        for b in range(w.B):
            for t in range(w.q_len):
                vis = int(lens[b]) - w.q_len + t + 1
                n = min(KT, vis)
                topk[b, t, :n] = torch.randperm(vis, generator=g, device=dev)[:n].to(torch.int32)
        plans = []
        for r in range(N):
            rows_t = torch.empty((w.B, w.q_len * KT), dtype=torch.int32, device=dev)
            plans.append((rows_t, torch.empty_like(rows_t), torch.empty(w.B, dtype=torch.int32, device=dev)))
    sinks = None
    if args.sinks:
        g = torch.Generator().manual_seed(7)
        sinks = torch.randn(w.H, generator=g).to(dev)
    for r, a in enumerate(attn_args):
        a.window, a.softcap = args.window, args.softcap
        if plans is not None:
            a.sparse_rows, a.sparse_bits, a.sparse_count = (x.data_ptr() for x in plans[r])
            a.sparse_stride = int(plans[r][0].shape[1])
        a.sinks = sinks.data_ptr() if sinks is not None and r == N - 1 else None
        a.q, a.pool = q.data_ptr(), sp.pools[r].data_ptr()
        a.block_table, a.seq_len = sp.tables[r].data_ptr(), sp.seq_len.data_ptr()
        ws_r = workspaces[r % args.streams]
        a.workspace, a.workspace_bytes = ws_r.data_ptr(), ws_r.numel()
        if args.records:
            a.o, a.lse = recs[r].data_ptr(), None
        else:
            a.o, a.lse = o_parts[r * K].data_ptr(), lse_parts[r * K].data_ptr()
        a.status = status.data_ptr()
    refs = [ctypes.byref(a) for a in attn_args]
    if multi_arr is not None:
        for r, a in enumerate(attn_args):
            multi_arr[r] = a
    sh = stream.cuda_stream
    rows = w.B * M

    def merge(sh_m):
        if args.records:
            rc = L.dcp_merge_heads(N, rows, 512, recs.data_ptr(), base, o.data_ptr(), lse.data_ptr(), sh_m)
        else:
            fn = L.dcp_lse_merge_bf16 if args.o_bf16 else L.dcp_lse_merge
            rc = fn(N * K, rows, 512, o_parts.data_ptr(), lse_parts.data_ptr(), base, o.data_ptr(),
                                 lse.data_ptr(), sh_m)
        if rc != 0:
            raise RuntimeError(f"merge: {dcp.strerror(rc)}")

    def one_launch_step(events=None, sh=sh):
        # events (3): before the launch, after it, after the merge -- nothing
        # else is recorded inside the step (each event costs GPU time)
        if events is not None:
            events[0].record(stream)
        rc = L.dcp_stripe_attn_multi(multi_arr, N, sh)
        if rc != 0:
            raise RuntimeError(f"dcp_stripe_attn_multi: {dcp.strerror(rc)}")
        if events is not None:
            events[1].record(stream)
        merge(sh)
        if events is not None:
            events[2].record(stream)

    def step(events=None, sh=sh):
        if multi_arr is not None:
            one_launch_step(events, sh)
            return
        per_rank_step(events, sh)

    def per_rank_step(events=None, sh=sh):
        # events (N + 2): before each rank's call, after the last call, after the merge
        two = len(streams) > 1
        if two:
            if events is not None:
                events[0].record(stream)
            # fork: the second stream starts after everything queued before the step
            fork = torch.cuda.Event()
            fork.record(stream)
            streams[1].wait_event(fork)
        for r in range(N):
            sh_r = streams[r % len(streams)].cuda_stream if two else sh
            if events is not None and not two:
                events[r].record(stream)
            if plans is not None:
                rc = L.dcp_sparse_plan(lay, r, w.B, w.q_len, args.topk, topk.data_ptr(), sp.seq_len.data_ptr(),
                                       plans[r][0].data_ptr(), plans[r][1].data_ptr(), plans[r][2].data_ptr(),
                                       int(plans[r][0].shape[1]), sh_r)
                if rc != 0:
                    raise RuntimeError(f"dcp_sparse_plan: {dcp.strerror(rc)}")
            rc = L.dcp_stripe_attn(refs[r], sh_r)
            if rc != 0:
                raise RuntimeError(f"dcp_stripe_attn: {dcp.strerror(rc)}")
        if two:
            join = torch.cuda.Event()
            join.record(streams[1])
            stream.wait_event(join)
        if events is not None:
            events[N].record(stream)
        merge(sh)
        if events is not None:
            events[N + 1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if int(status.item()) != 0:
        raise RuntimeError(f"device status {int(status.item())}")
    graph = None
    if args.graph:
        # every call of one step as one graph (the library allocates, clears
        # and synchronises nothing inside a call); replays run on `stream`
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream(dev)
        cap.wait_stream(stream)
        with torch.cuda.graph(graph, stream=cap):
            step(sh=cap.cuda_stream)
        stream.wait_stream(cap)
        for _ in range(2):
            graph.replay()
        torch.cuda.synchronize()

    flush_mib = args.flush_mib
    if flush_mib < 0:
        flush_mib = 1024 if float(lens.sum()) * ROW_BYTES < (1 << 30) else 0
    scratch = torch.empty((flush_mib << 20) // 4, dtype=torch.float32, device=dev) if flush_mib > 0 else None
    # event slots: the step's start, the end of its attention launches, the end of the merge
    e_att = 1 if args.multi else N
    e_end = e_att + 1
    evs = [[timing_event() for _ in range(e_end + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for k in range(args.steps):
        if scratch is not None:
            scratch.fill_(float(k))              # evicts the KV from the caches, outside the step's events
        if graph is not None:
            evs[k][0].record(stream)
            graph.replay()
            evs[k][e_att].record(stream)
            evs[k][e_end].record(stream)
        else:
            step(evs[k])
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t_start

    # ---- secondary variant: the same step with all N stripes in one launch
    # (the N-fold parallelism of one GPU), timed the same way
    one_launch = None
    if not (args.no_secondary or args.multi or args.streams > 1 or args.graph or args.topk > 0):
        arr2 = (dcp.dcp_attn_args * N)(*[dcp.dcp_attn_args.from_buffer_copy(a) for a in attn_args])
        need2 = ctypes.c_size_t(0)
        assert L.dcp_stripe_attn_multi_workspace(arr2, N, ctypes.byref(need2)) == 0
        ws2 = torch.empty(max(need2.value, 16), dtype=torch.uint8, device=dev)
        arr2[0].workspace, arr2[0].workspace_bytes = ws2.data_ptr(), ws2.numel()

        def step2(ev=None):
            if ev is not None:
                ev[0].record(stream)
            rc = L.dcp_stripe_attn_multi(arr2, N, sh)
            if rc != 0:
                raise RuntimeError(f"dcp_stripe_attn_multi: {dcp.strerror(rc)}")
            if ev is not None:
                ev[1].record(stream)
            merge(sh)
            if ev is not None:
                ev[2].record(stream)
        for _ in range(max(2, args.warmup // 2)):
            step2()
        ev2 = [[timing_event() for _ in range(3)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        for k in range(args.steps):
            if scratch is not None:
                scratch.fill_(float(k))
            step2(ev2[k])
        torch.cuda.synchronize()
        st2 = np.array([ev2[k][0].elapsed_time(ev2[k][2]) for k in range(args.steps)])
        la2 = np.array([ev2[k][0].elapsed_time(ev2[k][1]) for k in range(args.steps)])
        if int(status.item()) != 0:
            raise RuntimeError(f"device status {int(status.item())} after the one-launch step")
        one_launch = {"what": "the same step with the N stripe attentions in one dcp_stripe_attn_multi launch, "
                              "then the same merge (HIP-event step times)",
                      "us_per_step": round(float(st2.mean()) * 1e3, 1),
                      "us_per_step_median": round(float(np.median(st2)) * 1e3, 1),
                      "launch_us": round(float(la2.mean()) * 1e3, 1), "ms": float(st2.mean())}
        del ws2

    # ---- secondary form of a one-launch step: the per-rank form, N
    # dcp_stripe_attn calls (the launch each rank runs on its own GPU, with
    # its chunk combine) then the same merge, timed with an event per call
    per_rank = None
    if args.multi and not (args.no_secondary or args.graph):
        for _ in range(max(2, args.warmup // 2)):
            per_rank_step()
        ev3 = [[timing_event() for _ in range(N + 2)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        for k in range(args.steps):
            if scratch is not None:
                scratch.fill_(float(k))
            per_rank_step(ev3[k])
        torch.cuda.synchronize()
        if int(status.item()) != 0:
            raise RuntimeError(f"device status {int(status.item())} after the per-rank step")
        st3 = np.array([ev3[k][0].elapsed_time(ev3[k][N + 1]) for k in range(args.steps)])
        calls3 = np.array([[ev3[k][r].elapsed_time(ev3[k][r + 1]) for r in range(N)] for k in range(args.steps)])
        mg3 = np.array([ev3[k][N].elapsed_time(ev3[k][N + 1]) for k in range(args.steps)])
        per_rank = {"what": "the same step as N per-rank dcp_stripe_attn calls (each rank's launch and its chunk "
                            "combine, the shape one rank runs on its own GPU) on one stream, then the same merge "
                            "(HIP-event step times, one event per call)",
                    "us_per_step": round(float(st3.mean()) * 1e3, 1),
                    "us_per_step_median": round(float(np.median(st3)) * 1e3, 1),
                    "per_call_us": [round(float(x) * 1e3, 1) for x in calls3.mean(axis=0)],
                    "merge_us": round(float(mg3.mean()) * 1e3, 1),
                    "ms": float(st3.mean()), "call_ms": calls3.mean(axis=0)}

    power = None
    if args.power_seconds > 0:
        def loop_step():
            if scratch is not None:
                scratch.fill_(0.0)
            if graph is not None:
                graph.replay()
            else:
                step()
        power = sample_power(loop_step, args.power_seconds)

    if args.copy_calibration_mib > 0:
        # one plain elementwise pass of known size (reads n bytes, writes n
        # bytes) after the timed region: hardware byte counters of the
        # attention kernel are scaled by what they read for this kernel
        n = args.copy_calibration_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    if args.multi:
        # one launch of all stripes (with --graph: the whole graph's span, merge included)
        per_stripe_ms = np.array([[evs[k][0].elapsed_time(evs[k][1])] for k in range(args.steps)])
    elif args.streams > 1 or args.graph:
        # overlapping calls, or one graph, have no per-launch span: the stripe part of the step over N
        per_stripe_ms = np.array([[evs[k][0].elapsed_time(evs[k][N]) / N] * N for k in range(args.steps)])
    else:
        per_stripe_ms = np.array([[evs[k][r].elapsed_time(evs[k][r + 1]) for r in range(N)] for k in range(args.steps)])
    merge_ms = np.array([evs[k][e_att].elapsed_time(evs[k][e_end]) for k in range(args.steps)])
    step_ev_ms = np.array([evs[k][0].elapsed_time(evs[k][e_end]) for k in range(args.steps)])
    ms_per_step = wall_s * 1e3 / args.steps
    if scratch is not None:
        ms_per_step = float(step_ev_ms.mean())        # the flushes between steps are not step time

    # ---- algorithmic work
    local = counts.astype(np.int64)                                  # rows per (request, rank)
    if args.topk > 0:
        # rows the selection reaches on each rank (the plan's counts)
        local = np.stack([plans[r][2].cpu().numpy() for r in range(N)], axis=1).astype(np.int64)
    elif args.window > 0:
        # rows some query of the request sees: the last S - first window start
        first = np.clip(lens - w.q_len + 1 - args.window, 0, None)
        local = local - dcp.dcp_local_count(lay, torch.from_numpy(first.astype(np.int64)).to(dev)).cpu().numpy()
    kv_bytes = float(local.sum()) * ROW_BYTES
    for sec in (one_launch, per_rank):
        if sec is not None:
            ms2 = sec.pop("ms")
            sec["value"] = round(kv_bytes / (ms2 * 1e-3) / 1e9, 2)
            sec["unit"] = "GB/s"
            sec["hbm_frac"] = round(kv_bytes / (ms2 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    q_bytes = w.B * M * ROW_BYTES
    # per (row, head): a bf16 record, bf16 o + fp32 lse, or fp32 o + fp32 lse
    out_row_bytes = 1032 if args.records else (512 * 2 + 4 if args.o_bf16 else (512 + 1) * 4)
    part_bytes = K * w.B * M * out_row_bytes                           # one stripe's (o_r, lse_r), or its K parts
    vis = np.zeros(w.B)
    for t in range(w.q_len):
        seen = np.minimum(lens, lens - w.q_len + t + 1).clip(min=0)
        if args.window > 0:
            seen = np.minimum(seen, args.window)
        if args.topk > 0:
            seen = np.minimum(seen, args.topk)
        vis += seen
    flops = float((vis * w.H).sum()) * FLOP_PER_ROW_QUERY
    kv_gbs = kv_bytes / (ms_per_step * 1e-3) / 1e9
    # dominant kernel: one stripe-attention launch (its algorithmic bytes: the
    # stripe's latent rows, the queries, and its (o_r, lse_r))
    stripe_bytes = stripe_call_bytes(local, w.B, M, K, out_row_bytes)             # per rank
    launch_ms = per_stripe_ms.mean(axis=0)                                        # per rank
    if args.multi:
        # one launch for all stripes: its bytes over its duration
        launch_ms = launch_ms[:1]
        achieved = float(stripe_bytes.sum() / (launch_ms[0] * 1e-3)) / 1e9
    else:
        achieved = float(np.mean(stripe_bytes / (launch_ms * 1e-3))) / 1e9
    # a variant: no committed counter record applies (records are kept per
    # step form and output type)
    outputs = "bf16 records" if args.records else ("o_r bf16, lse_r fp32" if args.o_bf16 else "fp32")
    secondary = bool(args.window or args.softcap or args.sinks or args.parts or args.splits or I != 1 or args.topk
                     or args.streams > 1 or args.graph or args.records)
    if per_rank is not None:
        call_ms = per_rank.pop("call_ms")
        call_gbs = float(np.mean(stripe_bytes / (call_ms * 1e-3))) / 1e9
        per_rank["call"] = {"what": "one dcp_stripe_attn call: stripe_attn_kernel + its chunk combine",
                            "achieved": round(call_gbs, 1), "unit": "GB/s",
                            "frac": round(call_gbs / HBM_PEAK_GBS, 4),
                            "bytes_per_call": int(stripe_bytes.mean()),
                            "traffic": measured_traffic(w.name, "per-rank", outputs) if not secondary else None}
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    # the same launch's matrix rate: each rank's share of the step's FLOPs
    # (in proportion to its latent rows) over its duration
    rows_r = np.asarray(local, dtype=np.float64).sum(axis=0)
    stripe_flops = flops * rows_r / max(rows_r.sum(), 1.0)
    if args.multi:
        achieved_tf = float(stripe_flops.sum() / (launch_ms[0] * 1e-3)) / 1e12
    else:
        achieved_tf = float(np.mean(stripe_flops / (launch_ms * 1e-3))) / 1e12
    mfma_bound = flops / max(kv_bytes, 1.0) > MFMA_BF16_PEAK_TFLOPS / (HBM_PEAK_GBS / 1e3)

    # ---- measured HBM read peak: the streaming-read probe over the same pools,
    # one launch per stripe's pool, in the step's back-to-back pattern
    probe = None
    # pools of a few MB (Tiny) stream in a launch's latency: no peak to measure there
    if not args.no_probe and kv_bytes >= (64 << 20):
        probe = probe_pools(args, sp.pools, N, stream, dev)
    mfma_peak = None
    if not args.no_probe and mfma_bound:
        # above the spec ridge the step is MFMA-bound: its rate against the MFMA probe's
        mfma_peak, _, _, _ = mfma_probe_steps(N, 5, 2, stream, dev)

    # ---- parity of the last timed step's outputs against the oracle
    check = sample is not None and not (args.window or args.softcap or args.sinks or args.parts or args.topk)
    cpu = None
    parity = None
    if check:
        if args.records:
            host_out = records_to_host(recs, o, lse, w)
        else:
            host_out = (o.cpu().numpy(), lse.cpu().numpy(), o_parts.cpu().float().numpy(), lse_parts.cpu().numpy())
        slot_bad = slot_map_mismatches(lay, lens[:len(sample)], sp.tables, N, I, P, dev)
        cpu, parity = cpu_oracle_leg(args, w, sample, N, I, host_out)
        parity["slot_map_mismatches"] = slot_bad
        parity["ok"] = parity["ok"] and slot_bad == 0

    out = {
        "metric": "us/decode-step and KV GB/s (% HBM peak) for stripe attn+merge, K3 shape, 1 GPU",
        "value": round(kv_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "us_per_step": round(ms_per_step * 1e3, 1),
        "hbm_frac": round(kv_gbs / HBM_PEAK_GBS, 4),
        "tflops": round(tflops, 2),
        "mfma_frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
        **({"mfma_measured_peak": round(mfma_peak, 1), "mfma_frac_of_measured": round(tflops / mfma_peak, 4)}
           if mfma_peak else {}),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "S": int(lens.max()), "H": w.H, "q_len": w.q_len, "N": N,
                   "interleave": I, "page_size": P, "lse_base": w.lse_base, "kv_bytes": int(kv_bytes),
                   "launches_per_step": N + 1,
                   **({"variant": {"window": args.window, "softcap": args.softcap, "sinks": bool(args.sinks)}}
                      if (args.window or args.softcap or args.sinks) else {}),
                   **({"unmerged_parts": K, "merged_parts": N * K} if args.parts > 0 else {}),
                   **({"outputs": "bf16 records + fp32 lse in head-owner order, merged by dcp_merge_heads"}
                      if args.records else {}),
                   **({"topk": args.topk, "plan_in_step": True} if args.topk > 0 else {}),
                   "form": ("one launch of all N stripes (dcp_stripe_attn_multi), then the merge" if args.multi
                            else "N per-rank dcp_stripe_attn calls, then the merge"),
                   **({"streams": args.streams} if args.streams > 1 else {}),
                   **({"hip_graph": True} if args.graph else {})},
        "per_stripe_us": [round(float(x) * 1e3, 1) for x in launch_ms],
        "merge_us": round(float(merge_ms.mean()) * 1e3, 1),
        "event_step_us": round(float(step_ev_ms.mean()) * 1e3, 1),
        "event_step_us_median": round(float(np.median(step_ev_ms)) * 1e3, 1),
        "event_step_us_min": round(float(step_ev_ms.min()) * 1e3, 1),
        "flush_mib_between_steps": flush_mib,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if secondary else measured_traffic(w.name, "one-launch" if args.multi
                                                                       else "per-rank", outputs),
                     "kernel": ("one dcp_stripe_attn_multi launch: all stripes"
                                + (" (in one HIP graph with the merge: the step's time)" if args.graph else "")
                                if args.multi else
                                (f"one dcp_stripe_attn call: stripe_attn_kernel writing {K} unmerged parts"
                                 if args.parts > 0 else "one dcp_stripe_attn call: stripe_attn_kernel + its chunk combine")
                                + (" (bf16 record outputs)" if args.records else "")
                                + (" (o_r in bf16)" if args.o_bf16 else "")
                                + (" (two streams: the step's stripe time over N, calls overlapping)"
                                   if args.streams > 1 else "")
                                + (" (one HIP graph per step: the step's time, merge included, over N)"
                                   if args.graph else "")),
                     "bytes_per_launch": int(stripe_bytes.sum() if args.multi else stripe_bytes.mean())},
        "cpu_baseline": cpu,
        "parity": parity,
        "step_algorithmic_bytes": int(kv_bytes + N * q_bytes + 2 * N * part_bytes + w.B * M * (512 + 1) * 4),
        "outputs": outputs,
        "device": device_ids(dev),
        "power": power,
        "one_launch_for_all_stripes": one_launch,
        "per_rank_form": per_rank,
        "setup_s": round(setup_s, 1),
    }
    if probe is not None:
        peak = probe["hot_gbs"]
        out["roofline"]["measured_peak"] = round(peak, 1)
        out["roofline"]["frac_of_measured"] = round(achieved / peak, 4)
        out["roofline"]["measured_peak_probe"] = probe
    if mfma_bound:
        # above the spec ridge (312.5 FLOP per byte) the launch is bound by the
        # matrix cores: its rate against the bf16 MFMA peaks, with the memory
        # view kept beside it
        hbm_view = {k: out["roofline"].pop(k) for k in ("achieved", "peak", "unit", "frac", "measured_peak",
                                                       "frac_of_measured", "measured_peak_probe")
                    if k in out["roofline"]}
        out["roofline"] = {"bound": "mfma", "achieved": round(achieved_tf, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                           "unit": "TFLOP/s", "frac": round(achieved_tf / MFMA_BF16_PEAK_TFLOPS, 4),
                           **({"measured_peak": round(mfma_peak, 1),
                               "frac_of_measured": round(achieved_tf / mfma_peak, 4)} if mfma_peak else {}),
                           "flops_per_launch": int(stripe_flops.sum() if args.multi else stripe_flops.mean()),
                           **{k: v for k, v in out["roofline"].items() if k != "bound"},
                           "hbm_view": hbm_view}
    print(json.dumps(out), flush=True)
    if parity is not None and not parity["ok"]:
        print("parity check against the oracle FAILED", file=sys.stderr)
        sys.exit(3)


def records_to_host(recs, o, lse, w):
    """Host copies in request order of a records step: the merged (o, lse),
    written in head-owner order [N][B*q_len][H/N], and every rank's (o_r,
    lse_r) decoded from its bf16 records."""
    import torch
    N = recs.shape[0]
    Hl = w.H // N

    def owner_to_request(x):                       # [N, B*q_len, Hl, ...] -> [B, q_len, H, ...]
        x = x.reshape((N, w.B * w.q_len, Hl) + tuple(x.shape[3:]))
        return x.permute((1, 0, 2) + tuple(range(3, x.dim()))).reshape((w.B, w.q_len, w.H) + tuple(x.shape[3:]))

    o_h = owner_to_request(o.view(N, w.B * w.q_len, Hl, 512)).cpu().numpy()
    lse_h = owner_to_request(lse.view(N, w.B * w.q_len, Hl)).cpu().numpy()
    r_cpu = recs.cpu()
    op = np.stack([owner_to_request(r_cpu[r, ..., :512].contiguous().view(torch.bfloat16).float()).numpy()
                   for r in range(N)])
    lp = np.stack([owner_to_request(r_cpu[r, ..., 512:514].contiguous().view(torch.float32)[..., 0]).numpy()
                   for r in range(N)])
    return o_h, lse_h, op, lp


def sample_power(loop_step, seconds: float, sync=None):
    """Loop the step for `seconds` while `amd-smi metric --power --clock`
    samples the socket power and the GFX clocks of every XCD (each sample
    takes about a second).  None when amd-smi is missing or lists no GPU;
    GPU 0 of amd-smi is taken as this device only when it lists one GPU."""
    import re
    import shutil
    import subprocess
    import threading
    if sync is None:
        import torch
        sync = torch.cuda.synchronize
    if shutil.which("amd-smi") is None:
        return None

    def query(extra):
        try:
            r = subprocess.run(["amd-smi"] + extra, capture_output=True, text=True, timeout=20)
            return r.stdout if r.returncode == 0 else None
        except (OSError, subprocess.SubprocessError):
            return None

    listing = query(["list"]) or ""
    n_gpus = len(re.findall(r"^GPU:\s*\d+", listing, re.M))
    if n_gpus != 1:
        return {"skipped": f"amd-smi lists {n_gpus} GPUs: cannot tell which one this process uses"}
    samples = []
    stop = threading.Event()

    def sampler():
        while not stop.is_set():
            txt = query(["metric", "-g", "0", "--power", "--clock"])
            if txt is None:
                continue
            pw = re.findall(r"SOCKET_POWER:\s*(\d+)", txt)
            gfx = re.findall(r"GFX_\d+:\s*\n\s*CLK:\s*(\d+)", txt)
            if pw and gfx:
                samples.append((time.perf_counter(), float(pw[0]), [float(x) for x in gfx]))

    th = threading.Thread(target=sampler, daemon=True)
    t0 = time.perf_counter()
    th.start()
    k = 0
    while time.perf_counter() - t0 < seconds:
        loop_step()
        k += 1
        if k % 64 == 0:
            sync()
    sync()
    t_end = time.perf_counter()
    stop.set()
    th.join(timeout=30)
    # samples taken while the loop ran, past its first half second (clocks settle)
    use = [x for x in samples if t0 + 0.5 <= x[0] <= t_end]
    if not use:
        return {"skipped": "no amd-smi sample inside the loop"}
    pw = np.array([x[1] for x in use])
    clk = np.array([np.mean(x[2]) for x in use])
    per_xcd = np.array([x[2] for x in use if len(x[2]) == len(use[0][2])])
    return {"tool": "amd-smi metric --power --clock", "loop_seconds": round(t_end - t0, 2), "steps": k,
            "samples": len(use), "socket_w_mean": round(float(pw.mean()), 1), "socket_w_max": round(float(pw.max()), 1),
            "gfx_mhz_per_xcd": [round(float(v), 1) for v in per_xcd.mean(axis=0)],
            "gfx_mhz_mean": round(float(clk.mean()), 1), "gfx_mhz_min": round(float(clk.min()), 1),
            "xcds": len(use[-1][2])}


def device_ids(dev):
    """GPU and software identifiers of the run."""
    import torch
    props = torch.cuda.get_device_properties(dev)
    rocm = None
    try:
        with open("/opt/rocm/.info/version") as f:
            rocm = f.read().strip()
    except OSError:
        pass
    return {"name": props.name, "arch": getattr(props, "gcnArchName", None), "cus": props.multi_processor_count,
            "hip_runtime": torch.version.hip, "rocm": rocm, "torch": torch.__version__}


def probe_pools(args, pools, N, stream, dev):
    """The streaming-read probe (16-byte direct-to-LDS non-temporal loads, the
    stripe kernel's loader without compute) over each stripe's pool, N launches
    per step like the step's N attention launches, warm-up then timed steps;
    returns the mean rate of the timed launches and that of the first step."""
    import torch
    from mla_context_kv_amd import probe as PR
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    mode = "lds1"
    grid = PR.grid_for(mode, cus)
    sink = PR.make_sink(mode, grid, dev)
    per = pools[0].numel() * pools[0].element_size()
    sh = stream.cuda_stream
    for _ in range(args.warmup):
        for r in range(N):
            PR.stream(pools[r], per, mode, grid, sink, sh)
    evs = [[timing_event() for _ in range(N + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    got = 0
    for k in range(args.steps):
        for r in range(N):
            evs[k][r].record(stream)
            got = PR.stream(pools[r], per, mode, grid, sink, sh)
        evs[k][N].record(stream)
    torch.cuda.synchronize()
    ms = np.array([[evs[k][r].elapsed_time(evs[k][r + 1]) for r in range(N)] for k in range(args.steps)])
    gbs = got / (ms * 1e-3) / 1e9
    return {"mode": PR.MODE_NOTES[mode], "bytes_per_launch": got, "launches": int(ms.size),
            "hot_gbs": float(gbs.mean()), "first_step_gbs": round(float(gbs[0].mean()), 1),
            "us_per_launch": round(float(ms.mean()) * 1e3, 1)}


def slot_map_mismatches(lay, lens, tables, N, I, P, dev):
    """Positions of the given requests whose (owner, row, slot) from
    dcp_slot_map differ from the oracle's simulated hand-out, over every rank."""
    from mla_context_kv_amd import dcp, stripes
    from oracle import layout as OL
    pos, req = stripes.positions_and_requests(lens, dev)
    pos_h, req_h = pos.cpu().numpy(), req.cpu().numpy()
    bad = 0
    for r in range(N):
        own, row, slot = dcp.dcp_slot_map(lay, r, pos, req, tables[r])
        o_ref, r_ref, s_ref = OL.slot_map(pos_h, req_h, N, I, P, r, tables[r].cpu().numpy())
        bad += int(((own.cpu().numpy() != o_ref) | (row.cpu().numpy() != r_ref)
                    | (slot.cpu().numpy() != s_ref)).sum())
    return bad


O_ABS, O_REL, LSE_ABS = 4e-3, 1e-2, 2e-3        # |o - o_ref| <= 4e-3 + 1e-2 |o_ref|, |lse - lse_ref| <= 2e-3


def cpu_oracle_leg(args, w, sample, N, I, host_out):
    """The float64 oracle on the sampled requests, timed on every core of this
    process's affinity mask (BLAS threads pinned to that count): its striped
    attention + merge (the timed baseline) and its unsharded attention beside
    it.  Outside the timed calls, every sampled request's merged (o, lse) and
    every rank's (o_r, lse_r) from the GPU's last step are checked against the
    oracle's, elementwise, at the parity bar."""
    from contextlib import nullcontext
    from oracle import attention as OA
    from oracle import layout as OL
    from mla_context_kv_amd import workloads
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=cores)
    except ImportError:                      # threadpoolctl missing: BLAS keeps its own count
        limiter = nullcontext()
    o_g, lse_g, op_g, lp_g = host_out
    cpu_s = full_s = 0.0
    sample_bytes = 0.0
    worst_excess_o = worst_stripe_excess_o = -np.inf
    worst_abs_o = worst_lse = worst_stripe_lse = 0.0
    with limiter:
        for b, (qt, kvt, S) in enumerate(sample):
            qb, kvb = qt.double().numpy(), kvt.double().numpy()
            t1 = time.perf_counter()
            lists = OL.stripe_positions(S, N, I)
            parts = [OA.stripe_attention(qb, kvb, S, lists[r], workloads.SCALE, chunk=65536) for r in range(N)]
            o_m, lse_m = OA.lse_merge(np.stack([p[0] for p in parts]),
                                      np.stack([OA.to_base(p[1], w.lse_base) for p in parts]), w.lse_base)
            cpu_s += time.perf_counter() - t1
            if not args.no_unsharded_baseline:
                t2 = time.perf_counter()
                OA.full_attention(qb, kvb, S, workloads.SCALE, chunk=65536)      # the unsharded definition
                full_s += time.perf_counter() - t2
            sample_bytes += S * ROW_BYTES
            # parity of this request (not timed)
            d = np.abs(o_g[b] - o_m)
            worst_excess_o = max(worst_excess_o, float((d - (O_ABS + O_REL * np.abs(o_m))).max()))
            worst_abs_o = max(worst_abs_o, float(d.max()))
            worst_lse = max(worst_lse, float(np.abs(lse_g[b] - lse_m).max()))
            for r in range(N):
                po, pl = parts[r][0], OA.to_base(parts[r][1], w.lse_base)
                seen = np.isfinite(pl)
                if (np.isfinite(lp_g[r, b]) != seen).any():
                    worst_stripe_lse = float("inf")            # an empty stripe must be empty on both sides
                    continue
                if seen.any():
                    ds = np.abs(op_g[r, b] - po)[seen]
                    worst_stripe_excess_o = max(worst_stripe_excess_o,
                                                float((ds - (O_ABS + O_REL * np.abs(po[seen]))).max()))
                    worst_stripe_lse = max(worst_stripe_lse, float(np.abs(lp_g[r, b] - pl)[seen].max()))
    cpu = {"value": round(sample_bytes / cpu_s / 1e9, 4), "unit": "GB/s", "cores": int(cores),
           "kind": "oracle", "seconds": round(cpu_s, 3),
           "sample": f"{len(sample)} of {w.B} requests ({int(sum(s[2] for s in sample))} tokens, {w.H} heads, "
                     f"q_len {w.q_len}): all {N} stripe attentions + LSE merge in float64 NumPy, "
                     f"BLAS threads pinned to the {cores} cores of the process affinity mask"}
    if full_s > 0:
        cpu["unsharded_seconds"] = round(full_s, 3)
        cpu["unsharded_value"] = round(sample_bytes / full_s / 1e9, 4)
    ok = worst_excess_o <= 0 and worst_lse <= LSE_ABS and worst_stripe_excess_o <= 0 and worst_stripe_lse <= LSE_ABS
    parity = {"requests_checked": len(sample), "of_requests": w.B, "stripes_checked": N,
              "max_abs_o": worst_abs_o, "max_excess_o": worst_excess_o, "max_abs_lse": worst_lse,
              "stripe_max_excess_o": worst_stripe_excess_o, "stripe_max_abs_lse": worst_stripe_lse,
              "bar": f"|o-o_ref| <= {O_ABS} + {O_REL}|o_ref|, |lse-lse_ref| <= {LSE_ABS} (lse base {w.lse_base})",
              "ok": bool(ok)}
    return cpu, parity


def run_stream(args):
    """The streaming-read probe alone, in every load mode: per mode, N launches
    per step each reading one K3-sized stripe pool (1.208 GB; 9.66 GB per step
    in all), warm-up then timed steps, mean rate of the timed launches and
    that of the first timed step."""
    import torch
    from mla_context_kv_amd import probe as PR
    dev = torch.device("cuda:0")
    w = workloads_k3()
    N = w.N
    per = w.B * (w.S // w.N) * ROW_BYTES                        # one stripe's KV at K3
    buf = torch.zeros((N, per // 2), dtype=torch.int16, device=dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    res = {}
    for mode in ("lds1", "lds4", "reg"):
        grid = PR.grid_for(mode, cus)
        sink = PR.make_sink(mode, grid, dev)
        for _ in range(args.warmup):
            for r in range(N):
                PR.stream(buf[r], per, mode, grid, sink, sh)
        evs = [[timing_event() for _ in range(N + 1)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        got = 0
        for k in range(args.steps):
            for r in range(N):
                evs[k][r].record(stream)
                got = PR.stream(buf[r], per, mode, grid, sink, sh)
            evs[k][N].record(stream)
        torch.cuda.synchronize()
        ms = np.array([[evs[k][r].elapsed_time(evs[k][r + 1]) for r in range(N)] for k in range(args.steps)])
        gbs = got / (ms * 1e-3) / 1e9
        res[mode] = {"what": PR.MODE_NOTES[mode], "grid": grid, "hot_gbs": round(float(gbs.mean()), 1),
                     "first_step_gbs": round(float(gbs[0].mean()), 1), "min_us": round(float(ms.min()) * 1e3, 1),
                     "mean_us": round(float(ms.mean()) * 1e3, 1), "max_us": round(float(ms.max()) * 1e3, 1)}
    best = max(v["hot_gbs"] for v in res.values())
    power = None
    if args.power_seconds > 0:
        # the stripe kernel's own load mode, looped while power and clocks are sampled
        grid = PR.grid_for("lds1", cus)
        sink = PR.make_sink("lds1", grid, dev)

        def loop_step():
            for r in range(N):
                PR.stream(buf[r], per, "lds1", grid, sink, sh)
        power = sample_power(loop_step, args.power_seconds)
        if isinstance(power, dict):
            power["mode"] = "lds1"
    out = {"metric": "streaming HBM read GB/s (measured peak), K3-sized stripe pools, 1 GPU",
           "value": best, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(float(np.mean([v["mean_us"] for v in res.values()])) * N / 1e3, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u8", "data": "synthetic",
           "config": {"workload": "streaming read", "bytes_per_launch": per, "launches_per_step": N},
           "modes": res, "frac_of_spec": round(best / HBM_PEAK_GBS, 4), "device": device_ids(dev), "power": power}
    print(json.dumps(out), flush=True)


MFMA_PROBE_ITERS = 1600          # about 200 us per launch at the clock a loaded chip holds


def mfma_probe_steps(N, steps, warmup, stream, dev):
    """N launches of the MFMA probe per step (the stripe step's pattern), one
    workgroup of 8 waves per CU; returns (mean TFLOP/s of the timed launches,
    that of the first timed step, mean launch microseconds, grid)."""
    import torch
    from mla_context_kv_amd import probe as PR
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    sink = PR.make_mfma_sink(cus, dev)
    sh = stream.cuda_stream
    for _ in range(warmup):
        for _ in range(N):
            PR.mfma(cus, MFMA_PROBE_ITERS, sink, sh)
    evs = [[timing_event() for _ in range(N + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    flops = 0
    for k in range(steps):
        for r in range(N):
            evs[k][r].record(stream)
            flops = PR.mfma(cus, MFMA_PROBE_ITERS, sink, sh)
        evs[k][N].record(stream)
    torch.cuda.synchronize()
    ms = np.array([[evs[k][r].elapsed_time(evs[k][r + 1]) for r in range(N)] for k in range(steps)])
    tf = flops / (ms * 1e-3) / 1e12
    return float(tf.mean()), float(tf[0].mean()), float(ms.mean() * 1e3), cus


def run_mfma(args):
    """The MFMA probe alone: per step 8 launches of ~200 us, every SIMD
    running 32x32x16 bf16 MFMAs on four independent accumulator chains (two
    waves per SIMD, as in the stripe kernel), no memory traffic."""
    import torch
    from mla_context_kv_amd import probe as PR
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    N = 8
    hot, first, us, grid = mfma_probe_steps(N, args.steps, args.warmup, stream, dev)
    power = None
    if args.power_seconds > 0:
        sink = PR.make_mfma_sink(grid, dev)

        def loop_step():
            for _ in range(N):
                PR.mfma(grid, MFMA_PROBE_ITERS, sink, stream.cuda_stream)
        power = sample_power(loop_step, args.power_seconds)
    out = {"metric": "bf16 MFMA TFLOP/s (measured peak), v_mfma_f32_32x32x16_bf16 on every SIMD, 1 GPU",
           "value": round(hot, 1), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(us * N / 1e3, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "mfma stream", "grid": grid, "waves_per_workgroup": 8, "chains_per_wave": 4,
                      "iters": MFMA_PROBE_ITERS, "launches_per_step": N},
           "first_step_tflops": round(first, 1), "launch_us": round(us, 1),
           "frac_of_spec": round(hot / MFMA_BF16_PEAK_TFLOPS, 4), "device": device_ids(dev), "power": power}
    print(json.dumps(out), flush=True)


def workloads_k3():
    from mla_context_kv_amd import workloads
    return workloads.WORKLOADS["k3"]


def run_head_return(args):
    """Head-return exchange at the workload's shape: each of the N ranks packs
    its (o_r, lse_r) by head owner (dcp_pack_heads) and each owner merges the N
    records of its H/N heads (dcp_merge_heads).  The all-to-all between them is
    a plain block transpose on one GPU and is not timed.  Inputs: seeded
    partial results of the right shape (their values do not change the work)."""
    import torch
    from mla_context_kv_amd import dcp, workloads
    dev = torch.device("cuda:0")
    w = workloads.WORKLOADS[args.workload]
    N, V = w.N, 512
    rows = w.B * w.q_len
    Hl = w.H // N
    g = torch.Generator(device=dev).manual_seed(5)
    o_r = [torch.randn((rows, w.H, V), generator=g, device=dev) for _ in range(N)]
    lse_r = [torch.randn((rows, w.H), generator=g, device=dev) * 4 for _ in range(N)]
    send = torch.empty((N, N, rows, Hl, V + 4), dtype=torch.int16, device=dev)
    recv = torch.empty((N, N, rows, Hl, V + 4), dtype=torch.int16, device=dev)
    o = torch.empty((N, rows, Hl, V), dtype=torch.float32, device=dev)
    lse = torch.empty((N, rows, Hl), dtype=torch.float32, device=dev)
    base = 1 if w.lse_base == "2" else 0
    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        for r in range(N):
            dcp.dcp_pack_heads(o_r[r], lse_r[r], N, send=send[r])
        if ev is not None:
            ev[0].record(stream)
        recv.copy_(send.transpose(0, 1))                     # the all-to-all, emulated (not timed)
        if ev is not None:
            ev[1].record(stream)
        for d in range(N):
            dcp.dcp_merge_heads(recv[d], base, o=o[d], lse=lse[d])
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    evs = [[timing_event() for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for k in range(args.steps):
        evs[k][0].record(stream)
        step(evs[k][1:])
    torch.cuda.synchronize()
    pack_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    merge_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in evs]))
    rec = V * 2 + 8
    pack_bytes = N * (rows * w.H * (V * 4 + 4) + rows * w.H * rec)         # read fp32 partials, write records
    merge_bytes = N * (N * rows * Hl * rec + rows * Hl * (V + 1) * 4)      # read N records per row, write o, lse
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import attention as OA
        n_rows = min(4 * w.q_len, rows)                        # 4 requests
        parts = [(o_r[r][:n_rows].cpu().numpy(), lse_r[r][:n_rows].cpu().numpy()) for r in range(N)]
        t1 = time.perf_counter()
        sends = [OA.pack_heads(po, pl, N) for po, pl in parts]
        for d in range(N):
            OA.unpack_merge(np.stack([sends[r][d] for r in range(N)]), w.lse_base)
        cpu_s = time.perf_counter() - t1
        nb = (pack_bytes + merge_bytes) * n_rows / rows
        cpu = {"value": round(nb / cpu_s / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
               "seconds": round(cpu_s, 3), "sample": f"{n_rows // w.q_len} of {w.B} requests: pack + merge in NumPy"}
    t_ms = pack_ms + merge_ms
    gbs = (pack_bytes + merge_bytes) / (t_ms * 1e-3) / 1e9
    out = {
        "metric": "head-return pack + owner merge GB/s (all N ranks, all-to-all excluded), 1 GPU",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(t_ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "op": "head-return", "B": w.B, "q_len": w.q_len, "H": w.H, "N": N,
                   "record_bytes": rec, "payload_bytes_per_rank": rows * w.H * rec},
        "pack_us_all_ranks": round(pack_ms * 1e3, 1), "merge_us_all_owners": round(merge_ms * 1e3, 1),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "N dcp_pack_heads + N dcp_merge_heads"},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def run_relayout(args):
    """Prefill-to-decode token relayout of the whole batch: the requests sit in
    dense 64-token source pages (random page order); one step moves every
    request into all N ranks' compact pools (N dcp_relayout calls).  Bytes:
    every latent row read once and written once."""
    import torch
    from mla_context_kv_amd import dcp, stripes, workloads
    dev = torch.device("cuda:0")
    w = workloads.WORKLOADS[args.workload]
    I, N, P = args.interleave, w.N, w.page_size
    lay = dcp.layout(N, I, P)
    lens = workloads.seq_lens(w)
    B, D = w.B, workloads.ROW_DIM
    t0 = time.perf_counter()
    src_need = -(-lens // P)
    src_cols = int(src_need.max())
    src_pages = int(src_need.sum())
    rng = np.random.default_rng(11)
    perm = rng.permutation(src_pages).astype(np.int32)
    src_bt = np.full((B, src_cols), -1, dtype=np.int32)
    k = 0
    for b in range(B):
        src_bt[b, :src_need[b]] = perm[k:k + src_need[b]]
        k += src_need[b]
    src = torch.empty((src_pages, P, D), dtype=torch.bfloat16, device=dev)
    for b in range(B):
        rows = workloads.make_request_kv(w, b, int(lens[b]), dev)
        pad = torch.zeros((int(src_need[b]) * P - int(lens[b]), D), dtype=torch.bfloat16, device=dev)
        idx = torch.from_numpy(src_bt[b, :src_need[b]].astype(np.int64)).to(dev)
        src.index_copy_(0, idx, torch.cat([rows, pad]).view(-1, P, D))
    counts = dcp.dcp_local_count(lay, torch.from_numpy(lens.astype(np.int64)).to(dev)).cpu().numpy()
    tables, pool_pages = workloads.make_block_tables(w, stripes.pages_from_counts(counts, P))
    pools = [torch.empty((pool_pages, P, D), dtype=torch.bfloat16, device=dev) for _ in range(N)]
    bts = [torch.from_numpy(t).to(dev) for t in tables]
    src_bt_d = torch.from_numpy(src_bt).to(dev)
    start = torch.zeros(B, dtype=torch.int64, device=dev)
    length = torch.from_numpy(lens.astype(np.int64)).to(dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t0
    stream = torch.cuda.current_stream(dev)

    def step(events=None):
        for r in range(N):
            if events is not None:
                events[r].record(stream)
            dcp.dcp_relayout(lay, r, src, src_bt_d, start, length, bts[r], pools[r], max_len=int(lens.max()),
                             status=status)
        if events is not None:
            events[N].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if int(status.item()) != 0:
        raise RuntimeError(f"device status {int(status.item())}")
    evs = [[timing_event() for _ in range(N + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t1) * 1e3 / args.steps
    per_call_ms = np.array([[evs[k][r].elapsed_time(evs[k][r + 1]) for r in range(N)] for k in range(args.steps)])
    moved = counts.sum(axis=0) * ROW_BYTES * 2                       # per rank: read + write
    achieved = float(np.mean(moved / (per_call_ms.mean(axis=0) * 1e-3))) / 1e9
    gbs = float(lens.sum()) * ROW_BYTES * 2 / (ms_per_step * 1e-3) / 1e9

    cpu = None
    if not args.no_cpu_baseline:
        from oracle import layout as OL
        n_req = min(4, B)
        cpu_s = 0.0
        nbytes = 0
        for b in range(n_req):
            # the request's source pages (bit patterns), renumbered 0..n-1: not timed
            src_b = src[torch.from_numpy(src_bt[b, :src_need[b]].astype(np.int64)).to(dev)].view(torch.int16)
            src16 = src_b.reshape(-1, D).cpu().numpy()
            local_bt = np.arange(src_need[b], dtype=np.int32)
            t3 = time.perf_counter()
            for r in range(N):
                dst = np.empty((int(-(-counts[b, r] // P)) * P, D), dtype=np.int16)
                _, s_sl, d_sl = OL.relayout_plan(0, int(lens[b]), N, I, r, local_bt, P,
                                                 np.arange(dst.shape[0] // P, dtype=np.int32), P)
                OL.relayout(dst, src16, s_sl, d_sl)
            cpu_s += time.perf_counter() - t3
            nbytes += int(lens[b]) * ROW_BYTES * 2
        cpu = {"value": round(nbytes / cpu_s / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
               "seconds": round(cpu_s, 3),
               "sample": f"{n_req} of {B} requests: plan + row copy into all {N} ranks' pools in NumPy"}

    out = {
        "metric": "prefill-to-decode token relayout GB/s (read + write), K3 batch into N rank pools, 1 GPU",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "op": "relayout", "B": B, "S": int(lens.max()), "N": N, "interleave": I,
                   "page_size": P, "bytes_moved": int(lens.sum()) * ROW_BYTES * 2},
        "per_call_us": [round(float(x) * 1e3, 1) for x in per_call_ms.mean(axis=0)],
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "one dcp_relayout call (relayout_kernel)"},
        "cpu_baseline": cpu,
        "setup_s": round(setup_s, 1),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
