"""Every output slot is written by every entry point (needs the GPU).

Outputs are filled with a sentinel bit pattern before each call, twice with two
different patterns: the two calls must return the same bits, no slot may keep a
sentinel, and every value must lie in its documented range (token ids in
[0, V) or -1, probabilities in [0, 1] or -1, ...).  This catches a slot that a
kernel forgets on some path, which preallocated (torch.empty) outputs would
otherwise hide.  The batches mix greedy and stochastic requests with long
drafts cut early (a greedy request with k = 40 rejected at position 3),
k = 0, runs kept to the end, an invalid stochastic token, and an inconsistent
num_draft.
"""
import sys

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"
SENTINELS = (0x5A5A5A5A, 0x13579BDF)


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _as_i32(pattern):
    return int(np.array([pattern], np.uint32).view(np.int32)[0])


def _filled(n, dtype, pattern):
    """n elements of `dtype` whose 32-bit words all hold `pattern`."""
    item = torch.empty(0, dtype=dtype).element_size()
    words = max(n * item // 4, 1)
    t = torch.full((words,), _as_i32(pattern), dtype=torch.int32, device=DEV)
    return t.view(dtype)[:n]


def _bits(t):
    return t.contiguous().view(torch.int32).cpu().numpy() if t.numel() else np.zeros(0, np.int32)


def _no_sentinel(name, t):
    b = _bits(t)
    for s in SENTINELS:
        left = np.flatnonzero(b == _as_i32(s))
        assert left.size == 0, f"{name}: slots {left[:8]} keep the sentinel"


def _mixed_batch(V=3000, dtype="bf16"):
    """Requests: greedy k=40 cut at 3; stochastic k=40 kept throughout (p = q);
    greedy k=0; stochastic k=0; stochastic k=6 random; greedy k=33 kept
    throughout; stochastic k=3 with an invalid token; greedy k=2 random."""
    rng = np.random.default_rng(77)
    ks = [40, 40, 0, 0, 6, 33, 3, 2]
    greedy = [1, 0, 1, 0, 0, 1, 0, 1]
    B, K = len(ks), sum(ks)
    off = np.concatenate([[0], np.cumsum(ks)])
    tgt = torch.as_tensor(rng.normal(0, 2, size=(K + B, V)).astype(np.float32))
    tgt = tgt.to(torch.bfloat16).to(torch.float32).numpy()
    drf = np.zeros((K, V), np.float32)
    toks = np.zeros(K, np.int64)
    for b in range(B):
        for i in range(ks[b]):
            t = tgt[off[b] + b + i]
            d = t + rng.normal(0, 1.0, size=V).astype(np.float32)
            if b in (0, 5):
                y = int(np.argmax(t))
                if b == 0 and i == 3:
                    y = (y + 1) % V
            elif b == 1:
                d = t.copy()                      # p = q: kept for every u < 1
                y = int(rng.integers(V))
            elif b == 6 and i == 1:
                y = V + 5                         # invalid stochastic token
            else:
                y = int(rng.integers(V))
            drf[off[b] + i] = d
            toks[off[b] + i] = y
    u = (rng.random(K) * 0.98).astype(np.float32)
    uf = rng.random(B).astype(np.float32)
    return synth.from_arrays(tgt, drf, toks, ks, greedy=greedy, temperature=0.9, u_accept=u,
                             u_final=uf, dtype=dtype, name="poison_mixed", device=DEV)


def _call_verify(sv, batch, pattern, *, sample, max_k=None, num_draft=None):
    nd = torch.as_tensor(batch.num_draft if num_draft is None else num_draft,
                         dtype=torch.int32, device=DEV)
    outs = dict(accepted_len=_filled(batch.B, torch.int32, pattern),
                out_tokens=_filled(batch.K + batch.B, torch.int32, pattern))
    if sample:
        outs.update(p_draft=_filled(batch.K, torch.float32, pattern),
                    q_draft=_filled(batch.K, torch.float32, pattern),
                    resid_mass=_filled(batch.B, torch.float32, pattern))
        gm = torch.as_tensor(batch.greedy, dtype=torch.uint8, device=DEV)
        sv.spec_verify_sample(batch.target, batch.draft, batch.tokens, nd, batch.temperature,
                              batch.u_accept, batch.u_final, greedy_mask=gm, max_k=max_k, **outs)
    else:
        sv.spec_verify_greedy(batch.target, batch.tokens, nd, max_k=max_k,
                              accepted_len=outs["accepted_len"], out_tokens=outs["out_tokens"])
    torch.cuda.synchronize()
    return outs


def _check_ranges(batch, o, sample):
    nd = batch.num_draft.astype(np.int64)
    acc = o["accepted_len"].cpu().numpy()
    out = o["out_tokens"].cpu().numpy()
    assert np.all((acc == -1) | ((acc >= 0) & (acc <= nd))), acc
    assert np.all((out == -1) | ((out >= 0) & (out < batch.V))), out
    if sample:
        for name in ("p_draft", "q_draft"):
            v = o[name].cpu().numpy()
            assert np.all((v == -1) | ((v >= 0) & (v <= 1))), (name, v)
        rm = o["resid_mass"].cpu().numpy()
        assert np.all((rm == -1) | (rm >= 0)), rm


PLANS = [("multi", 1, None), ("single", 2, None), ("early_exit", 0, 40)]


@pytest.mark.parametrize("plan,code,max_k", PLANS, ids=[p[0] for p in PLANS])
@pytest.mark.parametrize("sample", [True, False], ids=["sample", "greedy"])
def test_every_verification_slot_is_written(plan, code, max_k, sample):
    import draft_token_verification_row_amd as sv
    batch = _mixed_batch()
    _log(f"[poison] {plan} sample={sample} B={batch.B} K={batch.K} V={batch.V}")
    sv.spec_verify_set_launch_plan(code)
    try:
        runs = [_call_verify(sv, batch, p, sample=sample, max_k=max_k) for p in SENTINELS]
    finally:
        sv.spec_verify_set_launch_plan(0)
    for name in runs[0]:
        _no_sentinel(f"{plan} {name}", runs[0][name])
        assert np.array_equal(_bits(runs[0][name]), _bits(runs[1][name])), (plan, name)
    _check_ranges(batch, runs[0], sample)
    acc = runs[0]["accepted_len"].cpu().numpy()
    if sample:
        assert acc[0] == 3 and acc[1] == 40 and acc[5] == 33 and acc[6] == -1, acc
        p = runs[0]["p_draft"].cpu().numpy()
        assert np.all(p[0:40] == -1)              # greedy request: -1 at every position
    else:
        assert acc[0] == 3 and acc[5] == 33, acc


@pytest.mark.parametrize("plan,code,max_k", PLANS, ids=[p[0] for p in PLANS])
def test_inconsistent_num_draft_writes_minus_one_everywhere(plan, code, max_k):
    import draft_token_verification_row_amd as sv
    batch = _mixed_batch()
    bad = batch.num_draft.copy()
    bad[2] = 1                                   # sum(num_draft) != K
    sv.spec_verify_set_launch_plan(code)
    try:
        runs = [_call_verify(sv, batch, p, sample=True, max_k=max_k, num_draft=bad)
                for p in SENTINELS]
    finally:
        sv.spec_verify_set_launch_plan(0)
    for name, t in runs[0].items():
        v = t.cpu().numpy()
        assert np.all(v == -1), (plan, name, v)
        assert np.array_equal(_bits(t), _bits(runs[1][name]))


def test_workload_batches_write_every_slot():
    """The reduced workloads through the default plan."""
    import draft_token_verification_row_amd as sv
    for cfg, kw in ((5, dict(B=40, V=40000)), (3, dict(B=6, V=20011)), (4, dict(B=2, V=5000)),
                    (2, dict(B=24, V=32000))):
        batch = synth.make_batch(cfg, DEV, **kw)
        sample = batch.temperature is not None
        for max_k in (None, int(batch.num_draft.max())):
            runs = [_call_verify(sv, batch, p, sample=sample, max_k=max_k) for p in SENTINELS]
            for name in runs[0]:
                _no_sentinel(f"cfg{cfg} {name}", runs[0][name])
                assert np.array_equal(_bits(runs[0][name]), _bits(runs[1][name])), (cfg, name)
            _check_ranges(batch, runs[0], sample)


def test_accept_stats_tree_and_adaptive_write_every_slot():
    import draft_token_verification_row_amd as sv
    acc = torch.tensor([0, 3, -1, 7, 2], dtype=torch.int32, device=DEV)
    nd = torch.tensor([1, 5, 4, 7, 2], dtype=torch.int32, device=DEV)
    st = [sv.spec_verify_accept_stats(acc, nd, 9, out=_filled(13, torch.float64, p))
          for p in SENTINELS]
    torch.cuda.synchronize()
    assert np.array_equal(_bits(st[0]), _bits(st[1]))
    _no_sentinel("accept_stats", st[0])

    tb = synth.make_tree_batch(1, DEV, B=6)
    nn = torch.as_tensor(tb.num_nodes, dtype=torch.int32, device=DEV)
    for max_depth in (None, 12):
        runs = []
        for p in SENTINELS:
            a, pa, o = (_filled(tb.B, torch.int32, p), _filled(tb.N, torch.int32, p),
                        _filled(tb.N, torch.int32, p))
            sv.spec_verify_tree_greedy(tb.target, tb.parent, tb.tokens, nn, max_depth=max_depth,
                                       accepted_len=a, path_nodes=pa, out_tokens=o)
            torch.cuda.synchronize()
            runs.append((a, pa, o))
        for x, y in zip(*runs):
            _no_sentinel("tree", x)
            assert np.array_equal(_bits(x), _bits(y))

    ab = synth.make_adaptive_batch(B=24, N=7, V=100, device=DEV, with_rows=False)
    B, N = ab.conf.shape
    runs = []
    for p in SENTINELS:
        r = dict(num_draft=_filled(B, torch.int32, p), offsets=_filled(B + 1, torch.int32, p),
                 tokens=_filled(B * N, torch.int32, p), src=_filled(B * N, torch.int32, p),
                 progress=_filled(B, torch.float64, p))
        st = sv.lib().spec_verify_adaptive_length(
            B, N, ab.conf.data_ptr(), ab.cost.data_ptr(), ab.tokens.data_ptr(),
            r["num_draft"].data_ptr(), r["offsets"].data_ptr(), r["tokens"].data_ptr(),
            r["src"].data_ptr(), r["progress"].data_ptr(), torch.cuda.current_stream().cuda_stream)
        assert st == 0
        torch.cuda.synchronize()
        runs.append(r)
    kept = int(runs[0]["offsets"][B].item())
    for name in runs[0]:
        a, b = runs[0][name], runs[1][name]
        if name in ("tokens", "src"):            # only the first offsets[B] entries are outputs
            a, b = a[:kept], b[:kept]
        _no_sentinel(f"adaptive {name}", a)
        assert np.array_equal(_bits(a), _bits(b)), name
