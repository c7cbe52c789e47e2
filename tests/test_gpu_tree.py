"""Greedy token-tree verification on the GPU against the tree oracle (needs the GPU).

Every output is integer: accepted lengths, walked node indices and committed
tokens must equal the oracle's exactly, for the all-rows entry point and the
early-exit one alike.
"""
import json
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _depth_bound(tb) -> int:
    par = tb.parent.cpu().numpy()
    off = tb.offsets
    best = 0
    for b in range(tb.B):
        s, n = int(off[b]), int(tb.num_nodes[b])
        d = [0] * n
        for i in range(1, n):
            d[i] = d[par[s + i]] + 1
        best = max(best, max(d))
    return best


def _run(tb, max_depth=None):
    import draft_token_verification_row_amd as sv
    r = sv.verify_tree_batch(tb, max_depth=max_depth)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy().astype(np.int64) for k, v in r.items()}


def _same(got, ref, label):
    for k in ("accepted_len", "path_nodes", "out_tokens"):
        bad = np.flatnonzero(got[k] != ref[k])
        assert bad.size == 0, f"{label} {k} at {bad[:8]}: gpu {got[k][bad[:8]]} oracle {ref[k][bad[:8]]}"


def _padded(tb, ld):
    t = torch.full((tb.N, ld), float("nan"), dtype=tb.target.dtype, device=tb.target.device)
    t[:, :tb.V] = tb.target
    return synth.TreeBatch(name=tb.name + "_strided", B=tb.B, N=tb.N, V=tb.V, dtype=tb.dtype,
                           num_nodes=tb.num_nodes, parent=tb.parent, tokens=tb.tokens,
                           target=t[:, :tb.V])


CASES = [
    ("tiny_f32", 1, {}),
    ("budget32_bf16_V40003", 2, dict(B=8, V=40003)),
    ("budget32_f32_V70001", 2, dict(B=5, V=70001, dtype="f32")),
    ("ragged_many_trees", 1, dict(B=1500, V=300, nodes=(1, 40))),
    ("single_node_trees", 1, dict(B=40, V=5000, nodes=1)),
    ("deep_matches", 2, dict(B=6, V=3000, p_match=1.0, nodes=60)),
    ("chains_100_deep", 1, dict(B=4, V=500, p_match=1.0, nodes=100, branch=1)),
    ("binary_70_deep", 1, dict(B=5, V=700, p_match=1.0, nodes=70, branch=2)),
    ("tiny_vocab", 1, dict(B=50, V=8, nodes=(1, 6))),
]


@pytest.mark.parametrize("label,cfg,kw", CASES, ids=[c[0] for c in CASES])
def test_tree_parity(label, cfg, kw):
    _log(f"[tree] {label} cfg={cfg} {kw}")
    tb = synth.make_tree_batch(cfg, DEV, **kw)
    ref = oracle.tree_verify_batch(**synth.tree_as_numpy(tb))
    _same(_run(tb), ref, label + " all-rows")
    md = _depth_bound(tb)
    _same(_run(tb, max_depth=md), ref, label + " early-exit")
    _same(_run(tb, max_depth=md + 3), ref, label + " early-exit (+3 rounds)")
    _log(f"[tree] {label}: B={tb.B} N={tb.N} max depth {md} mean accepted "
         f"{ref['accepted_len'].mean():.2f}")


@pytest.mark.parametrize("ld_extra,dtype", [(3, "bf16"), (5, "f32"), (8, "bf16")])
def test_tree_strided_rows(ld_extra, dtype):
    tb = synth.make_tree_batch(2, DEV, B=4, V=20001, dtype=dtype)
    tp = _padded(tb, tb.V + ld_extra)
    ref = oracle.tree_verify_batch(**synth.tree_as_numpy(tb))
    _same(_run(tp), ref, "strided all-rows")
    _same(_run(tp, max_depth=_depth_bound(tb)), ref, "strided early-exit")


def test_tree_golden_on_gpu():
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "tree_walk_example.json")))
    parent, tokens = g["tree"]["parent"], g["tree"]["tokens"]
    n, V = len(parent), g["vocab_size"]
    for case in g["cases"]:
        rows = np.zeros((n, V), np.float32)
        rows[:, 0] = 1.0
        for k, v in case["rows"].items():
            rows[int(k)] = v
        for dt in ("f32", "bf16"):
            tb = synth.tree_from_arrays(rows, parent, tokens, [n], dtype=dt, device=DEV)
            for md in (None, 3):
                got = _run(tb, max_depth=md)
                a = case["accepted_len"]
                assert got["accepted_len"].tolist() == [a], (case["name"], dt, md)
                assert got["path_nodes"][:a + 1].tolist() == case["path"]
                assert got["out_tokens"][:a + 1].tolist() == case["committed"]
                assert np.all(got["path_nodes"][a + 1:] == -1) and np.all(got["out_tokens"][a + 1:] == -1)


def test_tree_input_errors():
    tb = synth.make_tree_batch(2, DEV, B=6, V=3000, p_match=1.0, nodes=20)
    ref = oracle.tree_verify_batch(**synth.tree_as_numpy(tb))
    md = _depth_bound(tb)
    # a parent pointing forward makes only that request invalid
    par = tb.parent.clone()
    off = tb.offsets
    par[int(off[2]) + 5] = 7
    bad = synth.TreeBatch(**{**tb.__dict__, "parent": par})
    want = oracle.tree_verify_batch(**synth.tree_as_numpy(bad))
    assert want["accepted_len"][2] == -1
    _same(_run(bad), want, "bad parent all-rows")
    _same(_run(bad, max_depth=md), want, "bad parent early-exit")
    # num_nodes inconsistent with N: everything -1
    import draft_token_verification_row_amd as sv
    nn = torch.as_tensor(tb.num_nodes, dtype=torch.int32, device=DEV)
    nn[0] += 1
    nn[1] -= 2
    for m in (None, md):
        acc, path, out = sv.spec_verify_tree_greedy(tb.target, tb.parent, tb.tokens, nn, max_depth=m)
        torch.cuda.synchronize()
        assert torch.all(acc == -1) and torch.all(path == -1) and torch.all(out == -1)
    # early exit with too small a bound: walks longer than it report -1, the rest are exact
    lim = int(ref["accepted_len"].min())
    got = _run(tb, max_depth=lim)
    for b in range(tb.B):
        s, n = int(off[b]), int(tb.num_nodes[b])
        if ref["accepted_len"][b] > lim:
            assert got["accepted_len"][b] == -1
            assert np.all(got["path_nodes"][s:s + n] == -1) and np.all(got["out_tokens"][s:s + n] == -1)
        else:
            assert got["accepted_len"][b] == ref["accepted_len"][b]
            assert np.array_equal(got["path_nodes"][s:s + n], ref["path_nodes"][s:s + n])
            assert np.array_equal(got["out_tokens"][s:s + n], ref["out_tokens"][s:s + n])
    assert (ref["accepted_len"] > lim).any() and (ref["accepted_len"] <= lim).any()


def test_tree_full_size():
    """The tree workload at its real shape (32 trees of 33 nodes, V = 151936 bf16),
    both entry points, every request against the oracle."""
    tb = synth.make_tree_batch(2, DEV)
    torch.cuda.synchronize()
    _log(f"[tree full] B={tb.B} N={tb.N} V={tb.V}")
    ref = oracle.tree_verify_batch(**synth.tree_as_numpy(tb))
    _same(_run(tb), ref, "full all-rows")
    _same(_run(tb, max_depth=_depth_bound(tb)), ref, "full early-exit")
    _log(f"[tree full] mean accepted {ref['accepted_len'].mean():.2f}")
