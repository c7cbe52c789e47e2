"""Early-exit verification (rows read only up to each request's cut) against the
fp64 oracle and against the all-rows entry points (needs the GPU).

Accepted lengths, committed tokens and residual masses follow the oracle's
rule of tests/parity.py; p(y), q(y) are compared at the tested positions
(every position up to and including the cut) and must be -1 elsewhere.
Against the all-rows path the outputs are bit-identical.
"""
import sys

import numpy as np
import pytest
import torch

import synth
from tests.parity import compare, run_hip, run_oracle

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _tested_positions(batch, acc):
    """Boolean [K]: draft position i of request b was tested (stochastic, i <= a_b)."""
    nd = batch.num_draft.astype(np.int64)
    mask = np.zeros(int(nd.sum()), bool)
    off = np.concatenate([[0], np.cumsum(nd)])
    for b in range(batch.B):
        if batch.temperature is None or batch.greedy[b] or acc[b] < 0:
            continue
        n = min(int(acc[b]) + 1, int(nd[b]))
        mask[off[b]:off[b] + n] = True
    return mask


def _oracle_as_tested(batch, got, ref):
    """The oracle's p, q restricted to the positions the early-exit call tested."""
    if ref.get("p_draft") is None or got.get("p_draft") is None:
        return ref
    r = dict(ref)
    mask = _tested_positions(batch, got["accepted_len"])
    r["p_draft"] = np.where(mask, ref["p_draft"], -1.0)
    r["q_draft"] = np.where(mask, ref["q_draft"], -1.0)
    return r


def _assert_same_as_all_rows(batch, got, full, label):
    assert np.array_equal(got["accepted_len"], full["accepted_len"]), label
    assert np.array_equal(got["out_tokens"], full["out_tokens"]), label
    if got.get("resid_mass") is not None:
        assert np.array_equal(got["resid_mass"], full["resid_mass"]), label
        mask = _tested_positions(batch, got["accepted_len"])
        for name in ("p_draft", "q_draft"):
            assert np.array_equal(got[name][mask], full[name][mask]), (label, name)
            assert np.all(got[name][~mask] == -1.0), (label, name)


CASES = [
    ("tiny_full", 1, {}, 0),
    ("greedy_full", 2, {}, 0),
    ("f32_V40003", 3, dict(B=8, V=40003), 0),
    ("block16_bf16_V151936", 4, dict(B=3), 3),
    ("mixed_V70001", 5, dict(B=24, V=70001), 0),
    ("mixed_strided_scalar", 5, dict(B=12, V=9999, target_ld=10001), 1),
    ("k0_all_mixed", 5, dict(B=16, V=20000, k=0), 0),
    ("block16_tiny_vocab", 4, dict(B=64, V=64), 0),
    ("f32_vocab_1", 3, dict(B=4, V=1, k=2), 0),
    ("mixed_many_requests", 5, dict(B=2100, V=300), 2),
    ("greedy_odd_V", 2, dict(B=40, V=33333), 5),
]


@pytest.mark.parametrize("label,cfg,kw,extra", CASES, ids=[c[0] for c in CASES])
def test_early_exit_parity(label, cfg, kw, extra):
    """max_k = the largest k_b plus `extra` empty rounds."""
    _log(f"[early-exit] {label} cfg={cfg} {kw} extra={extra}")
    batch = synth.make_batch(cfg, DEV, **kw)
    max_k = int(batch.num_draft.max(initial=0)) + extra
    got = run_hip(batch, max_k=max_k)
    ref = run_oracle(batch)
    near = compare(batch, got, _oracle_as_tested(batch, got, ref), label)
    full = run_hip(batch)
    _assert_same_as_all_rows(batch, got, full, label)
    n_stoch = int((batch.greedy == 0).sum()) if batch.temperature is not None else 0
    _log(f"[early-exit] {label}: B={batch.B} K={batch.K} max_k={max_k} near_ties={near}")


def test_early_exit_largest_bound():
    """max_k = 4096 (the largest bound): thirteen windows, the last 2048 wide,
    on a batch whose requests are all decided in the first few."""
    batch = synth.make_batch(5, DEV, B=30, V=7000)
    got = run_hip(batch, max_k=4096)
    full = run_hip(batch)
    _assert_same_as_all_rows(batch, got, full, "max_k=4096")


def test_early_exit_count_above_bound_is_an_input_error():
    import draft_token_verification_row_amd as sv
    batch = synth.make_batch(5, DEV, B=10, V=5000)
    nd = torch.as_tensor(batch.num_draft, dtype=torch.int32, device=DEV)
    gm = torch.as_tensor(batch.greedy, dtype=torch.uint8, device=DEV)
    kmax = int(batch.num_draft.max())
    r = sv.spec_verify_sample(batch.target, batch.draft, batch.tokens, nd, batch.temperature,
                              batch.u_accept, batch.u_final, greedy_mask=gm, max_k=kmax - 1)
    torch.cuda.synchronize()
    assert torch.all(r["accepted_len"] == -1) and torch.all(r["out_tokens"] == -1)
    assert torch.all(r["p_draft"] == -1) and torch.all(r["resid_mass"] == -1)
    # the same workspace then serves a valid call
    r = sv.spec_verify_sample(batch.target, batch.draft, batch.tokens, nd, batch.temperature,
                              batch.u_accept, batch.u_final, greedy_mask=gm, max_k=kmax)
    torch.cuda.synchronize()
    assert torch.all(r["accepted_len"] >= 0)
    with pytest.raises(sv.SpecVerifyError):
        sv.spec_verify_greedy(batch.target, batch.tokens, nd, max_k=-1)
    with pytest.raises(sv.SpecVerifyError):
        sv.spec_verify_greedy(batch.target, batch.tokens, nd, max_k=4097)


def test_early_exit_invalid_token_marks_only_its_request():
    import draft_token_verification_row_amd as sv
    batch = synth.make_batch(5, DEV, B=10, V=5000)
    nd = torch.as_tensor(batch.num_draft, dtype=torch.int32, device=DEV)
    gm = torch.as_tensor(batch.greedy, dtype=torch.uint8, device=DEV)
    cand = np.flatnonzero((batch.greedy == 0) & (batch.num_draft > 1))
    b0 = int(cand[0])
    off = batch.offsets
    toks = batch.tokens.clone()
    toks[int(off[b0]) + int(batch.num_draft[b0]) - 1] = -3     # last draft: past any cut
    r = sv.spec_verify_sample(batch.target, batch.draft, toks, nd, batch.temperature,
                              batch.u_accept, batch.u_final, greedy_mask=gm,
                              max_k=int(batch.num_draft.max()))
    torch.cuda.synchronize()
    acc = r["accepted_len"].cpu().numpy()
    assert acc[b0] == -1
    sl = slice(int(off[b0]) + b0, int(off[b0]) + b0 + int(batch.num_draft[b0]) + 1)
    assert np.all(r["out_tokens"].cpu().numpy()[sl] == -1)
    dsl = slice(int(off[b0]), int(off[b0]) + int(batch.num_draft[b0]))
    assert np.all(r["p_draft"].cpu().numpy()[dsl] == -1)
    good = synth.select_requests(batch, [b for b in range(batch.B) if b != b0], device=DEV)
    ref = run_oracle(good)
    assert np.array_equal(np.delete(acc, b0), ref["accepted_len"])


def test_early_exit_repeat_and_stream():
    batch = synth.make_batch(5, DEV, B=64, V=30000)
    mk = int(batch.num_draft.max())
    a = run_hip(batch, max_k=mk)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        b = run_hip(batch, max_k=mk, stream=s)
    s.synchronize()
    for k in a:
        if a[k] is not None:
            assert np.array_equal(a[k], b[k]), k


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_early_exit_full_size(cfg):
    """Full workload shape in the launch configuration the benchmark times:
    bit-identical to the all-rows path, and every request against the oracle."""
    _log(f"[early-exit full] cfg={cfg} generating")
    batch = synth.make_batch(cfg, DEV)
    torch.cuda.synchronize()
    max_k = int(batch.num_draft.max())
    _log(f"[early-exit full] cfg={cfg} B={batch.B} K={batch.K} V={batch.V} max_k={max_k}")
    got = run_hip(batch, max_k=max_k)
    full = run_hip(batch)
    _assert_same_as_all_rows(batch, got, full, f"full cfg{cfg}")
    ref = run_oracle(batch, chunk=32)
    near = compare(batch, got, _oracle_as_tested(batch, got, ref), f"early-exit full cfg{cfg}")
    _log(f"[early-exit full] cfg={cfg}: {batch.B} requests, near_ties={near}")


@pytest.mark.parametrize("extra", [0, 70])
def test_early_exit_long_runs_span_wide_windows(extra):
    """Requests that keep long runs of drafts reach the late windows, up to 64
    positions wide (two 32-position chunks of the deciding wavefront): p = q on
    every stochastic position (kept for any u < 1), greedy drafts equal to the
    target argmax, and one forced cut per kind of request deep in a window."""
    rng = np.random.default_rng(123)
    V = 257
    ks = [0, 1, 31, 32, 33, 64, 100, 130, 70, 45]
    greedy = [0, 1, 0, 1, 0, 1, 0, 1, 0, 1]
    cut = {8: 69, 9: 40}
    B, K = len(ks), sum(ks)
    off = np.concatenate([[0], np.cumsum(ks)])
    tgt = torch.as_tensor(rng.normal(0, 2, size=(K + B, V)).astype(np.float32))
    tgt = tgt.to(torch.bfloat16).to(torch.float32).numpy()       # values bf16 holds exactly
    drf = np.zeros((K, V), np.float32)
    toks = np.zeros(K, np.int64)
    for b in range(B):
        for i in range(ks[b]):
            t = tgt[off[b] + b + i]
            d = t.copy()
            if greedy[b]:
                y = int(np.argmax(t))
                if cut.get(b) == i:
                    y = (y + 1) % V
            else:
                y = int(rng.integers(V))
                if cut.get(b) == i:
                    y = int(np.argmin(t))
                    d[y] = float(t.max()) + 8.0      # q(y) ~ 1, p(y) tiny: rejected
            drf[off[b] + i] = d
            toks[off[b] + i] = y
    u = (rng.random(K) * 0.9 + 0.05).astype(np.float32)
    uf = rng.random(B).astype(np.float32)
    batch = synth.from_arrays(tgt, drf, toks, ks, greedy=greedy, temperature=1.0, u_accept=u,
                              u_final=uf, dtype="bf16", name="long_runs", device=DEV)
    max_k = max(ks) + extra
    _log(f"[early-exit] long runs, max_k={max_k}")
    got = run_hip(batch, max_k=max_k)
    full = run_hip(batch)
    _assert_same_as_all_rows(batch, got, full, "long runs")
    want = [cut.get(b, ks[b]) for b in range(B)]
    assert got["accepted_len"].tolist() == want, got["accepted_len"]
    ref = run_oracle(batch)
    compare(batch, got, _oracle_as_tested(batch, got, ref), "long runs")
