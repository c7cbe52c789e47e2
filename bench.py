#!/usr/bin/env python3
"""Benchmark of one verification step on one MI355X.

A step is one call of the C ABI (all kernels: plan, row statistics, decide,
residual sweep, final draw) over one resident batch of synthetic logits.  The
default workload is the ragged mixed batch (B=512, k_b uniform in 0..7,
V=262144, bf16 logits, odd requests greedy, even requests stochastic at
T=0.8), the only workload that exercises every step of the path.

Prints ONE JSON line.  `value` = verified draft positions per second (sum of
k_b per step / step time).  `roofline` describes the row-statistics kernel:
algorithmic bytes (every logit row it must read, once) over its average
duration measured with HIP events recorded around it on the call's stream.
`other_path` times the other entry point (early exit vs all rows) on the same
batch.  `--workload tree` measures greedy token-tree verification instead (32
trees of 33 nodes over V = 151936 bf16; positions = draft nodes), and
`--workload adaptive` the confidence-driven length choice plus the gather of
the kept draft rows (512 blocks of 7 over V = 262144 bf16).  `cpu_baseline` times the fp64 oracle on a bounded sample of the same
workload.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verified draft positions/sec and achieved HBM GB/s vs peak (1× MI355X)"
PEAK_HBM_GBS = 8000.0
WORKLOADS = {"c1": 1, "c2": 2, "c3": 3, "c4": 4, "c5": 5, "tree": "tree", "adaptive": "adaptive"}
CSRC = os.path.join(ROOT, "draft_token_verification_row_amd", "csrc")
TRAFFIC = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_source_hash() -> str:
    """sha256 over the library sources (name and bytes of each csrc file, sorted)."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".hpp")):
            h.update(name.encode())
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(f.read())
    return h.hexdigest()[:16]


class HipEvents:
    """hipEvent_t handles from the HIP runtime the process already uses."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so.7")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def record(self, ev, stream):
        assert self.lib.hipEventRecord(ev, stream) == 0

    def create(self, n):
        evs = []
        for _ in range(n):
            e = ctypes.c_void_p()
            assert self.lib.hipEventCreate(ctypes.byref(e)) == 0
            evs.append(e.value)
        return evs

    def elapsed_ms(self, a, b) -> float:
        assert self.lib.hipEventSynchronize(b) == 0
        ms = ctypes.c_float()
        assert self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return float(ms.value)

    def destroy(self, evs):
        for e in evs:
            self.lib.hipEventDestroy(e)


def early_exit_windows(max_k: int):
    """Position windows [lo, hi) of the early-exit rounds the library launches
    for this max_k: 0, 1, 2, 4, 8, ... up to max_k + 1."""
    end = int(max_k) + 1
    out, lo, r = [], 0, 0
    while lo < end:
        hi = min(1 << r, end)
        out.append((lo, hi))
        lo, r = hi, r + 1
    return out


def early_exit_rows_read(acc, num_draft, stochastic, max_k: int) -> int:
    """Logit rows an early-exit call streams for row statistics, given its
    outcome: every row of the windows up to the one that holds each cut."""
    wins = early_exit_windows(max_k)
    total = 0
    for a, k, st in zip(acc, num_draft, stochastic):
        a, k = int(a), int(k)
        if a < 0:
            continue
        hi = next(h for (lo, h) in wins if lo <= a < h)
        total += min(hi, k + 1) + (min(hi, k) if st else 0)
    return total


def host_cpu() -> str:
    """CPU model and logical core count of the machine the oracle runs on."""
    model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return f"{model}, {os.cpu_count()} logical cores (the oracle used 1)"


def cpu_baseline(batch, min_seconds: float, max_requests: int):
    """The oracle as it stands, on the first requests of the batch, until at
    least `min_seconds` of CPU time have been spent (or `max_requests`)."""
    import synth
    import oracle
    done_pos = 0
    done_req = 0
    rows = 0
    t_total = 0.0
    step = 16
    while done_req < min(batch.B, max_requests) and t_total < min_seconds:
        reqs = list(range(done_req, min(done_req + step, batch.B)))
        sub = synth.select_requests(batch, reqs, device="cpu")
        d = synth.as_numpy(sub)
        t0 = time.perf_counter()
        oracle.verify_batch(**d)
        t_total += time.perf_counter() - t0
        done_pos += int(sub.num_draft.sum())
        rows += sub.K + sub.B + int(sub.num_draft[sub.greedy == 0].sum()) if sub.temperature else sub.K + sub.B
        done_req += len(reqs)
    return dict(value=done_pos / t_total if t_total > 0 else None, unit="verified draft positions/s",
                cores=1, kind="oracle", host=host_cpu(),
                sample=f"first {done_req} of {batch.B} requests ({done_pos} positions, {rows} logit rows), "
                       f"{t_total:.1f} s of fp64 NumPy on one host core")


def cpu_baseline_tree(tb, min_seconds: float):
    """The tree oracle as it stands, on the first requests, until `min_seconds`."""
    import synth
    import oracle
    done = nodes = 0
    t_total = 0.0
    while done < tb.B and t_total < min_seconds:
        reqs = list(range(done, min(done + 4, tb.B)))
        sub = synth.select_trees(tb, reqs, device="cpu")
        d = synth.tree_as_numpy(sub)
        t0 = time.perf_counter()
        oracle.tree_verify_batch(**d)
        t_total += time.perf_counter() - t0
        nodes += int(sub.num_nodes.sum()) - sub.B
        done += len(reqs)
    return dict(value=nodes / t_total if t_total > 0 else None, unit="verified draft positions/s",
                cores=1, kind="oracle", host=host_cpu(),
                sample=f"first {done} of {tb.B} trees ({nodes} draft nodes), {t_total:.1f} s of "
                       f"NumPy on one host core")


def bench_tree(args, sv, torch):
    """Greedy token-tree verification on the tree workload (32 trees of 33 nodes,
    V = 151936 bf16): headline = all node rows read once, other_path = early exit."""
    import synth
    dev = torch.device("cuda:0")
    tb = synth.make_tree_batch(2, dev)
    nn = torch.as_tensor(tb.num_nodes, dtype=torch.int32, device=dev)
    acc = torch.empty(tb.B, dtype=torch.int32, device=dev)
    path = torch.empty(tb.N, dtype=torch.int32, device=dev)
    out = torch.empty(tb.N, dtype=torch.int32, device=dev)
    wsb = sv.spec_verify_tree_workspace_bytes(tb.B, tb.N, tb.V)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    tr = sv.make_tree_struct(tb.target, tb.parent, tb.tokens, nn)
    sh = torch.cuda.current_stream().cuda_stream
    par = tb.parent.cpu().numpy()
    off = tb.offsets
    depth = 0
    for b in range(tb.B):
        d = [0] * int(tb.num_nodes[b])
        for i in range(1, len(d)):
            d[i] = d[par[int(off[b]) + i]] + 1
        depth = max(depth, max(d))
    lib = sv.lib()
    ptrs = (acc.data_ptr(), path.data_ptr(), out.data_ptr(), ws.data_ptr(), wsb, sh)
    calls = {False: lambda: lib.spec_verify_tree_greedy(ctypes.byref(tr), *ptrs),
             True: lambda: lib.spec_verify_tree_greedy_early_exit(ctypes.byref(tr), depth, *ptrs)}
    ee = args.early_exit
    for _ in range(args.warmup):
        assert calls[ee]() == 0
    torch.cuda.synchronize()
    if args.profile_only:
        for _ in range(args.steps):
            assert calls[ee]() == 0
        torch.cuda.synchronize()
        print(f"profile-only: {args.warmup + args.steps} calls of {tb.name}", flush=True)
        return
    hip = HipEvents()

    def timed(fn, steps):
        ev_b, ev_e = hip.create(steps), hip.create(steps)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            sv.spec_verify_set_profile_events(ev_b[i], ev_e[i])
            fn()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        sv.spec_verify_set_profile_events(None, None)
        ms = [hip.elapsed_ms(ev_b[i], ev_e[i]) for i in range(steps)]
        hip.destroy(ev_b + ev_e)
        return (t1 - t0) / steps, float(np.mean(ms)) / 1e3

    es = 4 if tb.dtype == "f32" else 2

    def rows_read(early_exit):
        if not early_exit:
            return tb.N
        # per round: each walk's current node and its descendants down to the
        # window's last step (the rows the round streams)
        a_np = acc.cpu().numpy().astype(np.int64)
        p_np = path.cpu().numpy().astype(np.int64)
        total = 0
        for b in range(tb.B):
            o, n = int(off[b]), int(tb.num_nodes[b])
            for lo, hi in early_exit_windows(depth):
                if a_np[b] < 0 or lo > a_np[b]:
                    break
                c = int(p_np[o + lo])
                cnt = 1
                for i in range(c + 1, n):
                    q = i
                    for _ in range(hi - lo - 1):
                        q = int(par[o + q])
                        if q <= c:
                            cnt += q == c
                            break
                total += cnt
        return total

    step_s, t_k = timed(calls[ee], args.steps)
    bytes_k = rows_read(ee) * tb.V * es
    for _ in range(max(args.warmup // 2, 2)):
        assert calls[not ee]() == 0
    o_step, o_t = timed(calls[not ee], max(args.steps // 2, 5))
    o_bytes = rows_read(not ee) * tb.V * es
    calls[ee]()
    torch.cuda.synchronize()
    positions = tb.N - tb.B
    achieved = bytes_k / t_k / 1e9
    traffic = None
    if os.path.exists(TRAFFIC):
        with open(TRAFFIC) as f:
            entry = json.load(f).get(tb.name + ("/early_exit" if ee else ""))
        if entry and entry.get("source_hash") == kernel_source_hash():
            traffic = entry.get("hbm_bytes_per_launch")
    path_name = lambda e: f"early exit (max_depth = {depth})" if e else "all node rows"
    a_np = acc.cpu().numpy()
    res = {
        "metric": METRIC, "value": positions / step_s, "unit": "verified draft positions/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": step_s * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": tb.name, "B": tb.B, "N": tb.N, "V": tb.V, "logits": tb.dtype,
                   "requests": "greedy token trees", "parallelism": "single GPU",
                   "path": path_name(ee)},
        "hbm_gbs_step": bytes_k / step_s / 1e9,
        "roofline": {"kernel": ("rounds: k_tree_round + k_tree_step_round per step" if ee
                                else "k_stats (argmax units of every node row)"),
                     "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
                     "algorithmic_bytes_per_launch": bytes_k, "avg_kernel_ms": t_k * 1e3},
        "other_path": {"path": path_name(not ee), "value": positions / o_step,
                       "ms_per_step": o_step * 1e3, "logit_bytes_read": o_bytes,
                       "hbm_gbs_step": o_bytes / o_step / 1e9, "timed_interval_ms": o_t * 1e3,
                       "speedup_of_headline": o_step / step_s},
        "acceptance": {"mean_accepted_nodes": float(a_np.mean()), "max_accepted": int(a_np.max())},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_tree(tb, args.cpu_seconds)
    print(json.dumps(res), flush=True)


def bench_adaptive(args, sv, torch):
    """Confidence-driven verification length for 512 requests with blocks of 7
    drafts over V = 262144 bf16 draft rows: one step = choose every k_b, pack the
    kept tokens, gather the kept draft rows into the packed layout."""
    import synth
    import oracle
    dev = torch.device("cuda:0")
    ab = synth.make_adaptive_batch(B=512, N=7, V=262144, dtype="bf16", device=dev)
    B, N, V = ab.B, ab.N, ab.V
    lib = sv.lib()
    nd = torch.empty(B, dtype=torch.int32, device=dev)
    off = torch.empty(B + 1, dtype=torch.int32, device=dev)
    toks = torch.empty(B * N, dtype=torch.int32, device=dev)
    src = torch.empty(B * N, dtype=torch.int32, device=dev)
    prog = torch.empty(B, dtype=torch.float64, device=dev)
    out = torch.empty(B * N, V, dtype=ab.draft.dtype, device=dev)
    sh = torch.cuda.current_stream().cuda_stream
    cnt = off[B:]

    def step():
        assert lib.spec_verify_adaptive_length(B, N, ab.conf.data_ptr(), ab.cost.data_ptr(),
                                               ab.tokens.data_ptr(), nd.data_ptr(), off.data_ptr(),
                                               toks.data_ptr(), src.data_ptr(), prog.data_ptr(), sh) == 0
        assert lib.spec_verify_gather_rows(1, V, ab.draft.data_ptr(), V, B * N, src.data_ptr(),
                                           cnt.data_ptr(), B * N, out.data_ptr(), V, sh) == 0

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.profile_only:
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        print(f"profile-only: {args.warmup + args.steps} steps of {ab.name}", flush=True)
        return
    hip = HipEvents()
    ev_b, ev_e = hip.create(args.steps), hip.create(args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        sv.spec_verify_set_profile_events(ev_b[i], ev_e[i])
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    sv.spec_verify_set_profile_events(None, None)
    g_ms = float(np.mean([hip.elapsed_ms(ev_b[i], ev_e[i]) for i in range(args.steps)]))
    hip.destroy(ev_b + ev_e)
    step_s = (t1 - t0) / args.steps
    K = int(off[B].item())
    bytes_g = 2 * K * V * 2                   # each kept row read once and written once
    achieved = bytes_g / (g_ms / 1e3) / 1e9
    traffic = None
    if os.path.exists(TRAFFIC):
        with open(TRAFFIC) as f:
            entry = json.load(f).get(ab.name)
        if entry and entry.get("source_hash") == kernel_source_hash():
            traffic = entry.get("hbm_bytes_per_launch")
    res = {
        "metric": METRIC, "value": K / step_s, "unit": "draft positions scheduled for verification/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": step_s * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f64",
        "data": "synthetic",
        "config": {"workload": ab.name, "B": B, "N": N, "V": V, "logits": ab.dtype,
                   "cost_table": ab.cost.cpu().numpy().tolist(), "kept_positions": K,
                   "parallelism": "single GPU"},
        "roofline": {"kernel": "k_gather_rows (kept draft rows into the packed layout)", "bound": "hbm",
                     "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
                     "algorithmic_bytes_per_launch": bytes_g, "avg_kernel_ms": g_ms},
        "mean_progress": float(prog.mean().item()),
    }
    if not args.no_cpu_baseline:
        c, co, tk = ab.conf.cpu().numpy(), ab.cost.cpu().numpy(), ab.tokens.cpu().numpy()
        t0 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t0 < args.cpu_seconds / 2 or reps == 0:
            oracle.adaptive_batch(c, co, tk)
            reps += 1
        dt = (time.perf_counter() - t0) / reps
        res["cpu_baseline"] = {"value": K / dt, "unit": res["unit"], "cores": 1, "kind": "oracle",
                               "sample": f"the whole selection and packing ({B} requests) x {reps}, "
                                         "no row gather (the oracle packs indices only)"}
    print(json.dumps(res), flush=True)


def copy_probe(mib: int, steps: int):
    """A plain copy kernel of known size: reads and writes mib MiB per launch."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.randn(n, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copy-probe: {steps} copies of {mib} MiB ({mib * 1024} KiB read + written each)", flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c5", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--profile-only", action="store_true",
                    help="run warmup+steps calls and exit without the JSON report (for rocprofv3)")
    ap.add_argument("--early-exit", action="store_true",
                    help="headline = the early-exit entry points (rows read only up to each cut); "
                         "the all-rows path is then reported under other_path, and vice versa")
    ap.add_argument("--mall-flush", choices=["auto", "on", "off"], default="auto",
                    help="write 512 MiB between timed calls so the 256 MB MALL holds no logits "
                         "(auto: on when one call reads less than 768 MiB)")
    ap.add_argument("--launch-plan", default="auto", choices=["auto", "multi", "single"],
                    help="launch plan of the all-rows entry points (library default: auto)")
    ap.add_argument("--shard", choices=["vocab", "request"], default=None,
                    help="run one GPU's share of the workload split over --shards GPUs: its "
                         "V/G columns (vocabulary-sharded logits) or its B/G requests")
    ap.add_argument("--shards", type=int, default=1, metavar="G")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="instead: run `steps` plain device copies of MIB MiB (counter calibration)")
    args = ap.parse_args()
    if args.copy_probe:
        return copy_probe(args.copy_probe, args.steps)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; the verification step of a "
                          "batch shards by request with no communication, so --gpus N > 1 is not "
                          "measured here", "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import torch
    import synth
    import draft_token_verification_row_amd as sv

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sv.spec_verify_set_launch_plan({"auto": 0, "multi": 1, "single": 2}[args.launch_plan])
    if args.workload == "tree":
        return bench_tree(args, sv, torch)
    if args.workload == "adaptive":
        return bench_adaptive(args, sv, torch)
    cfg_id = WORKLOADS[args.workload]
    shard_kw = {}
    if args.shard and args.shards > 1:
        full = synth.CONFIGS[cfg_id]
        shard_kw = {"V": full["V"] // args.shards} if args.shard == "vocab" \
            else {"B": max(1, full["B"] // args.shards)}
    batch = synth.make_batch(cfg_id, dev, **shard_kw)
    torch.cuda.synchronize()

    # Pre-built call: every buffer resident in HBM before timing.
    nd = torch.as_tensor(batch.num_draft, dtype=torch.int32, device=dev)
    gm = torch.as_tensor(batch.greedy, dtype=torch.uint8, device=dev) if batch.greedy.any() else None
    acc = torch.empty(batch.B, dtype=torch.int32, device=dev)
    out = torch.empty(batch.K + batch.B, dtype=torch.int32, device=dev)
    pdr = torch.empty(max(batch.K, 1), dtype=torch.float32, device=dev)
    qdr = torch.empty(max(batch.K, 1), dtype=torch.float32, device=dev)
    rm = torch.empty(batch.B, dtype=torch.float32, device=dev)
    ws_bytes = sv.spec_verify_workspace_bytes(batch.B, batch.K, batch.V)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    bt = sv.make_batch_struct(batch.target, batch.draft, batch.tokens, nd)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    lib = sv.lib()
    greedy_only = batch.temperature is None
    kmax = int(batch.num_draft.max()) if batch.K > 0 else 0

    def make_call(early_exit: bool):
        if greedy_only:
            if early_exit:
                return lambda: lib.spec_verify_greedy_early_exit(
                    ctypes.byref(bt), kmax, acc.data_ptr(), out.data_ptr(), ws.data_ptr(), ws_bytes, sh)
            return lambda: lib.spec_verify_greedy(ctypes.byref(bt), acc.data_ptr(), out.data_ptr(),
                                                  ws.data_ptr(), ws_bytes, sh)
        T = ctypes.c_float(batch.temperature)
        a_ptrs = (gm.data_ptr() if gm is not None else None, batch.u_accept.data_ptr(),
                  batch.u_final.data_ptr(), acc.data_ptr(), out.data_ptr(), pdr.data_ptr(),
                  qdr.data_ptr(), rm.data_ptr())
        if early_exit:
            return lambda: lib.spec_verify_sample_early_exit(ctypes.byref(bt), kmax, T, *a_ptrs,
                                                             ws.data_ptr(), ws_bytes, sh)
        return lambda: lib.spec_verify_sample(ctypes.byref(bt), T, *a_ptrs, ws.data_ptr(), ws_bytes, sh)

    ee = args.early_exit
    call = make_call(ee)
    for _ in range(args.warmup):
        assert call() == 0
    torch.cuda.synchronize()
    if args.profile_only:
        for _ in range(args.steps):
            assert call() == 0
        torch.cuda.synchronize()
        print(f"profile-only: {args.warmup + args.steps} calls of {batch.name}", flush=True)
        return

    hip = HipEvents()
    es = 4 if batch.dtype == "f32" else 2
    k_np = batch.num_draft.astype(np.int64)
    stoch = np.zeros(batch.B, bool) if greedy_only else (batch.greedy == 0)

    def rows_read(early_exit: bool) -> int:
        if not early_exit:      # every target row, the draft rows of stochastic requests
            return batch.K + batch.B + int(k_np[stoch].sum())
        # every row of the position windows up to the one holding each cut
        a_np = acc.cpu().numpy().astype(np.int64)
        return early_exit_rows_read(a_np, k_np, stoch, kmax)

    bytes_all = rows_read(False) * batch.V * es
    flush = args.mall_flush == "on" or (args.mall_flush == "auto" and bytes_all < (768 << 20))
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev) if flush else None

    def timed(fn, steps):
        """Per call: GPU time from HIP events around the C-ABI call on its stream
        (median, p10, p90), and the mean of the interval the library records
        around its row-statistics launches; plus wall time per call.  With the
        MALL flush a 512 MiB fill runs between calls, outside the call events."""
        ev_b, ev_e = hip.create(steps), hip.create(steps)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            if flush:
                scratch.zero_()
            sv.spec_verify_set_profile_events(ev_b[i], ev_e[i])
            fn()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        sv.spec_verify_set_profile_events(None, None)
        ms = [hip.elapsed_ms(ev_b[i], ev_e[i]) for i in range(steps)]
        hip.destroy(ev_b + ev_e)
        wall = (t1 - t0) / steps
        # per-call GPU time in a separate pass (events around each call would
        # slow the back-to-back loop above)
        n = min(steps, 50)
        cb, ce = hip.create(n), hip.create(n)
        for i in range(n):
            if flush:
                scratch.zero_()
            hip.record(cb[i], sh)
            fn()
            hip.record(ce[i], sh)
        torch.cuda.synchronize()
        call_ms = np.array([hip.elapsed_ms(cb[i], ce[i]) for i in range(n)])
        hip.destroy(cb + ce)
        step = float(np.median(call_ms)) / 1e3 if flush else wall
        return step, float(np.mean(ms)) / 1e3, call_ms, wall

    step_s, t_stats, call_ms, wall_s = timed(call, args.steps)
    positions = int(batch.num_draft.sum())
    rows = rows_read(ee)
    bytes_stats = rows * batch.V * es
    achieved = bytes_stats / t_stats / 1e9

    # the other entry point on the same batch, for comparison
    other = make_call(not ee)
    for _ in range(max(args.warmup // 2, 2)):
        assert other() == 0
    o_step, o_t, _, _ = timed(other, max(args.steps // 2, 5))
    o_bytes = rows_read(not ee) * batch.V * es
    call()                      # leave the headline path's outputs in acc/out
    torch.cuda.synchronize()

    traffic = None
    if os.path.exists(TRAFFIC):
        with open(TRAFFIC) as f:
            tr = json.load(f)
        entry = tr.get(batch.name if not ee else batch.name + "/early_exit")
        if entry and entry.get("source_hash") == kernel_source_hash():
            traffic = entry.get("hbm_bytes_per_launch")

    path = lambda e: ("early exit (max_k = %d)" % kmax) if e else "all rows"
    res = {
        "metric": METRIC,
        "value": positions / step_s,
        "unit": "verified draft positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_s * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": batch.name, "B": batch.B, "K": batch.K, "V": batch.V,
            "logits": batch.dtype, "temperature": batch.temperature,
            "requests": ("greedy" if greedy_only else
                         f"{int((batch.greedy == 1).sum())} greedy, {int((batch.greedy == 0).sum())} stochastic"),
            "parallelism": ("single GPU" if not shard_kw else
                            f"one GPU's share of a {args.shards}-way {args.shard} split"),
            "path": path(ee),
            "launch_plan": args.launch_plan,
        },
        "call_gpu_us": {"median": float(np.median(call_ms)) * 1e3,
                        "p10": float(np.percentile(call_ms, 10)) * 1e3,
                        "p90": float(np.percentile(call_ms, 90)) * 1e3,
                        "wall_per_call": wall_s * 1e6,
                        "timing": ("median of per-call HIP events, 512 MiB MALL flush between calls"
                                   if flush else "wall clock over back-to-back calls")},
        "rows_per_s": (batch.K + batch.B) / step_s,
        "hbm_gbs_step": bytes_stats / step_s / 1e9,
        "hbm_frac_step": bytes_stats / step_s / 1e9 / PEAK_HBM_GBS,
        "roofline": {
            "kernel": ("rounds: k_round + k_decide_round per position" if ee
                       else "k_stats (row statistics)"),
            "bound": "hbm",
            "achieved": achieved,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS,
            "traffic": traffic,
            "traffic_ratio": (traffic / bytes_stats) if traffic else None,
            "algorithmic_bytes_per_launch": bytes_stats,
            "avg_kernel_ms": t_stats * 1e3,
        },
        "other_path": {
            "path": path(not ee),
            "value": positions / o_step,
            "ms_per_step": o_step * 1e3,
            "logit_bytes_read": o_bytes,
            "hbm_gbs_step": o_bytes / o_step / 1e9,
            "timed_interval_ms": o_t * 1e3,
            "speedup_of_headline": o_step / step_s,
        },
    }
    st_out = torch.empty(4 + max(kmax, 1), dtype=torch.float64, device=dev)
    sv.spec_verify_accept_stats(acc, nd, max(kmax, 1), out=st_out)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(50):
        sv.spec_verify_accept_stats(acc, nd, max(kmax, 1), out=st_out)
    e1.record()
    torch.cuda.synchronize()
    st = st_out.cpu().numpy()
    res["acceptance"] = {
        "note": "from the timed calls' outputs; MAL counts the correction/bonus token, AR = kept/proposed drafts",
        "mean_kept_drafts": float(st[1]), "MAL": float(st[2]), "AR": float(st[3]),
        "per_position": [round(float(x), 4) for x in st[4:4 + max(kmax, 1)]],
        "stats_call_us": e0.elapsed_time(e1) * 1e3 / 50,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(batch, args.cpu_seconds, max_requests=batch.B)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
