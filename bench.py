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
batch.  `--workload ddtree_budget32_v151936` measures greedy token-tree verification instead (32
trees of 33 nodes over V = 151936 bf16; positions = draft nodes), and
`--workload adaptive_block7_v262144` the confidence-driven length choice plus the gather of
the kept draft rows (512 blocks of 7 over V = 262144 bf16).  `cpu_baseline` times the fp64 oracle on a bounded sample of the same
workload.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verified draft positions/sec and achieved HBM GB/s vs peak (1× MI355X)"
PEAK_HBM_GBS = 8000.0
WORKLOADS = {"tiny_stochastic": 1, "greedy_v32000": 2, "stochastic_f32_v128256": 3,
             "dflash_block16_v151936": 4, "ragged_mixed_v262144": 5,
             "ddtree_budget32_v151936": "tree", "adaptive_block7_v262144": "adaptive"}
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
    return f"{model}, {os.cpu_count()} logical cores visible"


def host_threads() -> int:
    """Host threads the oracle may use: the CPUs this process may run on, capped
    by OMP_NUM_THREADS when it is set (the GPU host's share of its CPUs)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, n)


def oracle_inputs(batch, chunk: int = 16):
    """Host copies of the batch in groups of `chunk` consecutive requests (the
    layout the oracle takes), made before any oracle timing starts."""
    import synth
    parts = []
    for s0 in range(0, batch.B, chunk):
        sub = synth.select_requests(batch, list(range(s0, min(s0 + chunk, batch.B))), device="cpu")
        parts.append(synth.as_numpy(sub))
    return parts


def run_oracle_timed(parts, threads: int, early_exit: bool):
    """The oracle as it stands on every group, serially or by a pool of threads
    over the groups (requests are independent; NumPy releases the GIL inside
    its array loops).  Returns (results concatenated in request order, seconds)."""
    import oracle
    from concurrent.futures import ThreadPoolExecutor

    def one(d):
        return oracle.verify_batch(**d, early_exit=early_exit)

    t0 = time.perf_counter()
    if threads <= 1:
        res = [one(d) for d in parts]
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            res = list(ex.map(one, parts))
    dt = time.perf_counter() - t0
    return {k: np.concatenate([r[k] for r in res]) for k in res[0]}, dt


def run_c_oracle_timed(batch, threads: int):
    """The fp64 C oracle as it stands on the whole batch (fp32 host copies;
    bf16 widens exactly), all-rows and early-exit forms, on one thread and on
    `threads`.  Returns (the all-rows result, {(form, threads): seconds})."""
    import synth
    import oracle.verify_c as vc
    d = synth.as_numpy(batch)
    vc.default()
    times, out = {}, None
    for form, ee in (("all_rows", False), ("early_exit", True)):
        for thr in sorted({1, threads}):
            t0 = time.perf_counter()
            r = vc.verify_batch(**d, early_exit=ee, threads=thr)
            times[(form, thr)] = time.perf_counter() - t0
            if form == "all_rows" and out is None:
                out = r
    del d
    return out, times


def oracles_agree(batch, c_res: dict, np_res: dict) -> bool:
    """The C and NumPy oracles on the same batch: equal accepted lengths and
    committed tokens, p(y), q(y) within 1e-12."""
    ok = (np.array_equal(c_res["accepted_len"], np_res["accepted_len"])
          and np.array_equal(c_res["out_tokens"], np_res["out_tokens"]))
    for key in ("p_draft", "q_draft"):
        if batch.K > 0:
            ok = ok and bool(np.all(np.abs(c_res[key] - np_res[key]) <= 1e-12))
    return bool(ok)


def parity_summary(batch, gpu: dict, ref: dict, near_tie: float = 1e-6) -> dict:
    """GPU outputs against the oracle's, per request: equal (accepted length,
    committed tokens), else a near-tie when the oracle's deciding margin is
    below 1e-6 relative, else a mismatch.  Also the largest |p(y) - p_oracle|
    and |q(y) - q_oracle| over the stochastic draft rows."""
    nd = batch.num_draft.astype(np.int64)
    off = np.concatenate([[0], np.cumsum(nd)])
    mism = near = 0
    for b in range(batch.B):
        sl = slice(int(off[b]) + b, int(off[b]) + b + int(nd[b]) + 1)
        if (int(gpu["accepted_len"][b]) == int(ref["accepted_len"][b])
                and np.array_equal(gpu["out_tokens"][sl].astype(np.int64), ref["out_tokens"][sl])):
            continue
        if not batch.greedy[b] and batch.temperature is not None and ref["margin"][b] < near_tie:
            near += 1
        else:
            mism += 1
    res = {"requests": int(batch.B), "mismatches": mism, "near_ties": near}
    if gpu.get("p_draft") is not None and batch.temperature is not None and batch.K > 0:
        rows = np.repeat(batch.greedy == 0, nd)
        if rows.any():
            for name in ("p_draft", "q_draft"):
                res[f"max_abs_err_{name[0]}"] = float(np.max(np.abs(
                    gpu[name][rows].astype(np.float64) - ref[name][rows])))
    return res


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


def read_probe(mib: int, steps: int, warmup: int):
    """The plain streaming read of the library (the access pattern of the
    row-statistics kernel without its arithmetic) over mib MiB: the read
    bandwidth ceiling, from the events the library records around its launch."""
    import torch
    import draft_token_verification_row_amd as sv
    src = torch.randn(mib * (1 << 20) // 4, device="cuda:0")
    sink = torch.zeros(64, dtype=torch.int32, device="cuda:0")
    for _ in range(warmup):
        sv.spec_verify_read_probe(src, sink)
    torch.cuda.synchronize()
    hip = HipEvents()
    eb, ee = hip.create(steps), hip.create(steps)
    for i in range(steps):
        sv.spec_verify_set_profile_events(eb[i], ee[i])
        sv.spec_verify_read_probe(src, sink)
    torch.cuda.synchronize()
    sv.spec_verify_set_profile_events(None, None)
    ms = np.array([hip.elapsed_ms(eb[i], ee[i]) for i in range(steps)])
    hip.destroy(eb + ee)
    nbytes = src.numel() * 4
    print(json.dumps({"read_probe_mib": mib, "steps": steps, "bytes": nbytes,
                      "mean_us": float(ms.mean()) * 1e3, "median_us": float(np.median(ms)) * 1e3,
                      "gbs_mean": nbytes / (ms.mean() / 1e3) / 1e9,
                      "gbs_median": nbytes / (np.median(ms) / 1e3) / 1e9,
                      "frac_of_8TBs": nbytes / (np.median(ms) / 1e3) / 1e9 / PEAK_HBM_GBS}), flush=True)


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
    ap.add_argument("--workload", default="ragged_mixed_v262144", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle (CPU baseline and parity against it)")
    ap.add_argument("--no-configs", action="store_true",
                    help="measure only the chosen workload (no `configs` object)")
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
    ap.add_argument("--read-probe", type=int, default=0, metavar="MIB",
                    help="instead: time the library's plain streaming read over MIB MiB")
    args = ap.parse_args()
    if args.copy_probe:
        return copy_probe(args.copy_probe, args.steps)
    if args.read_probe:
        return read_probe(args.read_probe, args.steps, args.warmup)

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
    if WORKLOADS[args.workload] == "tree":
        return bench_tree(args, sv, torch)
    if WORKLOADS[args.workload] == "adaptive":
        return bench_adaptive(args, sv, torch)
    cfg_id = WORKLOADS[args.workload]
    shard_kw = {}
    if args.shard and args.shards > 1:
        full = synth.CONFIGS[cfg_id]
        shard_kw = {"V": full["V"] // args.shards} if args.shard == "vocab" \
            else {"B": max(1, full["B"] // args.shards)}
    hip = HipEvents()
    head = VerifyWorkload(synth.make_batch(cfg_id, dev, **shard_kw), sv, torch, hip, args.mall_flush)
    if args.profile_only:
        head.profile_only(args.early_exit, args.warmup, args.steps)
        return
    res = head.report(args, args.early_exit, args.steps, args.warmup)
    if shard_kw:
        res["config"]["parallelism"] = f"one GPU's share of a {args.shards}-way {args.shard} split"

    # the oracle: parity of the headline outputs and the CPU baseline
    if not args.no_cpu_baseline:
        parts = oracle_inputs(head.batch)
        nthr = host_threads()
        ref1, t1 = run_oracle_timed(parts, 1, False)
        refn, tn = run_oracle_timed(parts, nthr, False)
        _, te1 = run_oracle_timed(parts, 1, True)
        _, ten = run_oracle_timed(parts, nthr, True)
        assert all(np.array_equal(ref1[k], refn[k]) for k in ("accepted_len", "out_tokens"))
        del parts
        try:
            cres, c_times = run_c_oracle_timed(head.batch, nthr)
            c_error = None
        except (OSError, RuntimeError, subprocess.CalledProcessError) as e:   # no C compiler or library
            cres, c_times, c_error = None, {}, f"{type(e).__name__}: {e}"
        pos = head.batch.K
        res["parity"] = parity_summary(head.batch, head.outputs(), ref1)
        res["parity"]["rule"] = ("every request of the timed batch against the fp64 oracle; a "
                                 "near-tie is a disagreement whose deciding margin is below 1e-6 "
                                 "relative")
        res["parity"]["c_oracle_agrees"] = (oracles_agree(head.batch, cres, ref1)
                                             if cres is not None else None)
        variants = {
            "numpy_all_rows_1_thread": {"value": pos / t1, "seconds": t1},
            f"numpy_all_rows_{nthr}_threads": {"value": pos / tn, "seconds": tn},
            "numpy_early_exit_1_thread": {"value": pos / te1, "seconds": te1},
            f"numpy_early_exit_{nthr}_threads": {"value": pos / ten, "seconds": ten},
        }
        for (form, thr), dt in c_times.items():
            variants[f"c_{form}_{thr}_{'thread' if thr == 1 else 'threads'}"] = {
                "value": pos / dt, "seconds": dt}
        c_all = c_times.get(("all_rows", nthr), float("inf"))
        best_c = c_all < tn
        res["cpu_baseline"] = {
            "value": pos / min(tn, c_all), "unit": "verified draft positions/s", "cores": nthr,
            "kind": "oracle", "host": host_cpu(),
            "sample": (f"all {head.batch.B} requests ({pos} positions) of the timed batch, all "
                       f"rows, {nthr} threads: the faster of the fp64 C oracle (OpenMP over "
                       f"requests) and the fp64 NumPy oracle (a thread pool over groups of 16 "
                       f"requests); this run: {'C' if best_c else 'NumPy'}"),
            "variants": variants,
        }
        if c_error:
            res["cpu_baseline"]["c_oracle_error"] = c_error

    # every workload, briefly (the headline's own entry reuses its numbers)
    if not args.no_configs and not shard_kw:
        configs = {}
        for cid in sorted(synth.CONFIGS):
            if cid == cfg_id:
                wl = head
                entry = wl.summary(res)
            else:
                wl = VerifyWorkload(synth.make_batch(cid, dev), sv, torch, hip, args.mall_flush)
                r = wl.report(args, False, min(args.steps, 50), min(args.warmup, 10),
                              with_other=True, acceptance=False)
                entry = wl.summary(r)
            if not args.no_cpu_baseline:
                if cid == cfg_id:
                    entry["parity"] = res["parity"]
                else:
                    ref, _ = run_oracle_timed(oracle_inputs(wl.batch), host_threads(), False)
                    entry["parity"] = parity_summary(wl.batch, wl.outputs(), ref)
            configs[wl.batch.name] = entry
            if wl is not head:
                wl.release()
        res["configs"] = configs
    print(json.dumps(res), flush=True)


class VerifyWorkload:
    """One resident verification batch with pre-built C-ABI calls."""

    def __init__(self, batch, sv, torch, hip, mall_flush):
        self.batch, self.sv, self.torch, self.hip = batch, sv, torch, hip
        dev = batch.target.device
        torch.cuda.synchronize()
        self.nd = torch.as_tensor(batch.num_draft, dtype=torch.int32, device=dev)
        self.gm = (torch.as_tensor(batch.greedy, dtype=torch.uint8, device=dev)
                   if batch.greedy.any() else None)
        self.acc = torch.empty(batch.B, dtype=torch.int32, device=dev)
        self.out = torch.empty(batch.K + batch.B, dtype=torch.int32, device=dev)
        self.pdr = torch.empty(max(batch.K, 1), dtype=torch.float32, device=dev)
        self.qdr = torch.empty(max(batch.K, 1), dtype=torch.float32, device=dev)
        self.rm = torch.empty(batch.B, dtype=torch.float32, device=dev)
        self.ws_bytes = sv.spec_verify_workspace_bytes(batch.B, batch.K, batch.V)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)
        self.bt = sv.make_batch_struct(batch.target, batch.draft, batch.tokens, self.nd)
        self.sh = torch.cuda.current_stream().cuda_stream
        self.greedy_only = batch.temperature is None
        self.kmax = int(batch.num_draft.max()) if batch.K > 0 else 0
        self.es = 4 if batch.dtype == "f32" else 2
        self.k_np = batch.num_draft.astype(np.int64)
        self.stoch = np.zeros(batch.B, bool) if self.greedy_only else (batch.greedy == 0)
        self.bytes_all = self.rows_read(False) * batch.V * self.es
        self.flush = mall_flush == "on" or (mall_flush == "auto" and self.bytes_all < (768 << 20))
        self.scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev) if self.flush else None

    def call(self, early_exit: bool):
        lib, bt, ws, wsb, sh = self.sv.lib(), self.bt, self.ws, self.ws_bytes, self.sh
        acc, out = self.acc.data_ptr(), self.out.data_ptr()
        if self.greedy_only:
            if early_exit:
                return lambda: lib.spec_verify_greedy_early_exit(
                    ctypes.byref(bt), self.kmax, acc, out, ws.data_ptr(), wsb, sh)
            return lambda: lib.spec_verify_greedy(ctypes.byref(bt), acc, out, ws.data_ptr(), wsb, sh)
        T = ctypes.c_float(self.batch.temperature)
        a_ptrs = (self.gm.data_ptr() if self.gm is not None else None,
                  self.batch.u_accept.data_ptr(), self.batch.u_final.data_ptr(), acc, out,
                  self.pdr.data_ptr(), self.qdr.data_ptr(), self.rm.data_ptr())
        if early_exit:
            return lambda: lib.spec_verify_sample_early_exit(ctypes.byref(bt), self.kmax, T,
                                                             *a_ptrs, ws.data_ptr(), wsb, sh)
        return lambda: lib.spec_verify_sample(ctypes.byref(bt), T, *a_ptrs, ws.data_ptr(), wsb, sh)

    def rows_read(self, early_exit: bool) -> int:
        b = self.batch
        if not early_exit:      # every target row, the draft rows of stochastic requests
            return b.K + b.B + int(self.k_np[self.stoch].sum())
        a_np = self.acc.cpu().numpy().astype(np.int64)
        return early_exit_rows_read(a_np, self.k_np, self.stoch, self.kmax)

    def profile_only(self, early_exit, warmup, steps):
        fn = self.call(early_exit)
        for _ in range(warmup + steps):
            assert fn() == 0
        self.torch.cuda.synchronize()
        print(f"profile-only: {warmup + steps} calls of {self.batch.name}", flush=True)

    def timed(self, fn, steps):
        """Wall clock over `steps` back-to-back calls with nothing else on the
        stream (a 512 MiB fill between calls when the MALL is flushed); then,
        in separate passes of up to 50 calls, the GPU time of each call from
        HIP events around it on its stream, and the duration of the
        row-statistics launch from the events the library records around it."""
        torch, hip, sh = self.torch, self.hip, self.sh
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            if self.flush:
                self.scratch.zero_()
            fn()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / steps
        n = min(steps, 50)
        cb, ce = hip.create(n), hip.create(n)
        for i in range(n):
            if self.flush:
                self.scratch.zero_()
            hip.record(cb[i], sh)
            fn()
            hip.record(ce[i], sh)
        torch.cuda.synchronize()
        call_ms = np.array([hip.elapsed_ms(cb[i], ce[i]) for i in range(n)])
        hip.destroy(cb + ce)
        eb, ee = hip.create(n), hip.create(n)
        for i in range(n):
            if self.flush:
                self.scratch.zero_()
            self.sv.spec_verify_set_profile_events(eb[i], ee[i])
            fn()
        torch.cuda.synchronize()
        self.sv.spec_verify_set_profile_events(None, None)
        stats_ms = [hip.elapsed_ms(eb[i], ee[i]) for i in range(n)]
        hip.destroy(eb + ee)
        step = float(np.median(call_ms)) / 1e3 if self.flush else wall
        return step, float(np.mean(stats_ms)) / 1e3, call_ms, wall

    def report(self, args, ee, steps, warmup, with_other=True, acceptance=True) -> dict:
        b = self.batch
        fn = self.call(ee)
        for _ in range(warmup):
            assert fn() == 0
        step_s, t_stats, call_ms, wall_s = self.timed(fn, steps)
        positions = int(b.num_draft.sum())
        bytes_stats = self.rows_read(ee) * b.V * self.es
        achieved = bytes_stats / t_stats / 1e9
        path = lambda e: ("early exit (max_k = %d)" % self.kmax) if e else "all rows"
        res = {
            "metric": METRIC, "value": positions / step_s, "unit": "verified draft positions/s",
            "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": step_s * 1e3,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
            "data": "synthetic",
            "config": {
                "workload": b.name, "B": b.B, "K": b.K, "V": b.V, "logits": b.dtype,
                "temperature": b.temperature,
                "requests": ("greedy" if self.greedy_only else
                             f"{int((b.greedy == 1).sum())} greedy, {int((b.greedy == 0).sum())} stochastic"),
                "parallelism": "single GPU", "path": path(ee), "launch_plan": args.launch_plan,
            },
            "call_gpu_us": {"median": float(np.median(call_ms)) * 1e3,
                            "p10": float(np.percentile(call_ms, 10)) * 1e3,
                            "p90": float(np.percentile(call_ms, 90)) * 1e3,
                            "wall_per_call": wall_s * 1e6,
                            "timing": ("median of per-call HIP events, 512 MiB MALL flush between calls"
                                       if self.flush else "wall clock over back-to-back calls")},
            "rows_per_s": (b.K + b.B) / step_s,
            "hbm_gbs_step": self.bytes_all / step_s / 1e9 if not ee else bytes_stats / step_s / 1e9,
            "hbm_frac_step": (self.bytes_all if not ee else bytes_stats) / step_s / 1e9 / PEAK_HBM_GBS,
            "roofline": {
                "kernel": ("rounds: k_round + k_decide_round per window" if ee
                           else "k_stats (row statistics)"),
                "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS, "traffic": self.traffic(ee),
                "algorithmic_bytes_per_launch": bytes_stats, "avg_kernel_ms": t_stats * 1e3,
            },
        }
        tr = res["roofline"]["traffic"]
        res["roofline"]["traffic_ratio"] = (tr / bytes_stats) if tr else None
        if with_other:
            other = self.call(not ee)
            for _ in range(max(warmup // 2, 2)):
                assert other() == 0
            o_step, o_t, _, _ = self.timed(other, max(steps // 2, 5))
            o_bytes = self.rows_read(not ee) * b.V * self.es
            res["other_path"] = {
                "path": path(not ee), "value": positions / o_step, "ms_per_step": o_step * 1e3,
                "logit_bytes_read": o_bytes, "hbm_gbs_step": o_bytes / o_step / 1e9,
                "timed_interval_ms": o_t * 1e3, "speedup_of_headline": o_step / step_s,
            }
        assert fn() == 0            # leave the headline path's outputs in the buffers
        self.torch.cuda.synchronize()
        if acceptance:
            res["acceptance"] = self.acceptance()
        return res

    def traffic(self, ee):
        if not os.path.exists(TRAFFIC):
            return None
        with open(TRAFFIC) as f:
            tr = json.load(f)
        entry = tr.get(self.batch.name if not ee else self.batch.name + "/early_exit")
        if entry and entry.get("source_hash") == kernel_source_hash():
            return entry.get("hbm_bytes_per_launch")
        return None

    def acceptance(self) -> dict:
        torch, sv = self.torch, self.sv
        kmax = max(self.kmax, 1)
        st_out = torch.empty(4 + kmax, dtype=torch.float64, device=self.acc.device)
        sv.spec_verify_accept_stats(self.acc, self.nd, kmax, out=st_out)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(50):
            sv.spec_verify_accept_stats(self.acc, self.nd, kmax, out=st_out)
        e1.record()
        torch.cuda.synchronize()
        st = st_out.cpu().numpy()
        return {
            "note": "from the timed calls' outputs; MAL counts the correction/bonus token, AR = kept/proposed drafts",
            "mean_kept_drafts": float(st[1]), "MAL": float(st[2]), "AR": float(st[3]),
            "per_position": [round(float(x), 4) for x in st[4:4 + kmax]],
            "stats_call_us": e0.elapsed_time(e1) * 1e3 / 50,
        }

    def outputs(self) -> dict:
        o = {"accepted_len": self.acc.cpu().numpy(), "out_tokens": self.out.cpu().numpy()}
        if not self.greedy_only:
            o.update(p_draft=self.pdr[:self.batch.K].cpu().numpy(),
                     q_draft=self.qdr[:self.batch.K].cpu().numpy(), resid_mass=self.rm.cpu().numpy())
        return o

    def summary(self, r: dict) -> dict:
        """The per-workload line of the `configs` object."""
        out = {
            "B": self.batch.B, "K": self.batch.K, "V": self.batch.V, "logits": self.batch.dtype,
            "step_us": r["ms_per_step"] * 1e3, "timing": r["call_gpu_us"]["timing"],
            "positions_per_s": r["value"], "bytes_all": self.bytes_all,
            "call_frac_of_8TBs": r["hbm_frac_step"],
            "k_stats_frac_of_8TBs": r["roofline"]["frac"], "k_stats_us": r["roofline"]["avg_kernel_ms"] * 1e3,
        }
        if "other_path" in r:
            out["early_exit_step_us"] = r["other_path"]["ms_per_step"] * 1e3
            out["early_exit_positions_per_s"] = r["other_path"]["value"]
        return out

    def release(self):
        self.batch = self.scratch = self.ws = None
        self.torch.cuda.empty_cache()


if __name__ == "__main__":
    main()
