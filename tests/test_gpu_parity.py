"""HIP path against the fp64 oracle, element by element (needs the GPU).

Small cases span several 32 KiB row units and ragged tails; full-size cases
run each workload at its real shape, in the same launch configuration the
benchmark times, and check a seeded sample of requests against the oracle
every request against the oracle, plus invariants that hold for every
request.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from tests import oracle_pins as pins
from tests.parity import compare, run_hip, run_oracle

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


SMALL = [
    ("tiny_full", 1, {}),
    ("greedy_full", 2, {}),
    ("f32_V40003", 3, dict(B=8, V=40003)),
    ("block16_bf16_V151936", 4, dict(B=3)),
    ("mixed_V70001", 5, dict(B=24, V=70001)),
    ("mixed_strided_vec", 5, dict(B=12, V=50000, target_ld=50048)),
    ("mixed_strided_scalar", 5, dict(B=12, V=9999, target_ld=10001)),
    ("f32_strided_scalar", 3, dict(B=6, V=4099, target_ld=4101)),
    ("k0_all_mixed", 5, dict(B=16, V=20000, k=0)),
    ("block16_tiny_vocab", 4, dict(B=64, V=64)),
    ("f32_vocab_1", 3, dict(B=4, V=1, k=2)),
    ("mixed_many_requests", 5, dict(B=2100, V=300)),
    ("greedy_odd_V", 2, dict(B=40, V=33333)),
    # more rows than k_stats plans in LDS (2K + B > 6144 with B <= 2048): the
    # separate plan kernel writes the row lists
    ("mixed_rows_beyond_lds_plan", 5, dict(B=600, V=3001, k=7)),
    ("f32_rows_beyond_lds_plan", 3, dict(B=400, V=2000, k=8)),
]


@pytest.mark.parametrize("label,cfg,kw", SMALL, ids=[s[0] for s in SMALL])
def test_small_parity(label, cfg, kw):
    _log(f"[parity] {label} cfg={cfg} {kw}")
    batch = synth.make_batch(cfg, DEV, **kw)
    got = run_hip(batch)
    ref = run_oracle(batch)
    near = compare(batch, got, ref, label)
    n_stoch = int((batch.greedy == 0).sum()) if batch.temperature is not None else 0
    _log(f"[parity] {label}: B={batch.B} K={batch.K} near_ties={near}")


def _golden_batch(rows_t, rows_d, toks, greedy, T, u, w):
    return synth.from_arrays(rows_t, rows_d, toks, [len(toks)], greedy=[greedy],
                             temperature=T, u_accept=u, u_final=[w], dtype="f32", device=DEV)


def test_golden_examples_on_gpu():
    g = pins.load_golden("abr_example.json")
    voc = {s: i for i, s in enumerate(g["vocab"])}
    tgt = pins._logits_from_probs(g["target_probs"])
    dr = pins._logits_from_probs(g["draft_probs"])
    toks = [voc[s] for s in g["draft_tokens"]]
    want = [voc[s] for s in g["expected"]["committed"]]
    for uC in (g["reject_threshold_C"] + 1e-6, 0.5, 0.99):
        for w in (0.0, 0.3, 0.999):
            b = _golden_batch(tgt, dr, toks, 0, 1.0, [0.3, 0.7, uC, 0.0], w)
            got = run_hip(b)
            assert got["accepted_len"][0] == 2
            assert got["out_tokens"][:3].tolist() == want and got["out_tokens"][3:].tolist() == [-1, -1]
    g = pins.load_golden("round_t1_t4.json")
    voc = {s: i for i, s in enumerate(g["vocab"])}
    tgt = pins._logits_from_probs(g["target_probs"])
    dr = pins._logits_from_probs(g["draft_probs"])
    toks = [voc[s] for s in g["draft_tokens"]]
    for w, name in g["expected"]["replacement_for_w"]:
        b = _golden_batch(tgt, dr, toks, 0, 1.0, [0.99, 0.99, 0.5, 0.0], w)
        got = run_hip(b)
        assert got["out_tokens"][:3].tolist() == [voc["T1"], voc["T2"], voc[name]], (w, got)
    g = pins.load_golden("weather_example.json")
    voc = {s: i for i, s in enumerate(g["vocab"])}
    b = synth.from_arrays(g["target_logits"], None, [voc[s] for s in g["draft_tokens"]], [4],
                          greedy=[1], dtype="bf16", device=DEV)
    got = run_hip(b)
    assert got["accepted_len"][0] == 2
    assert got["out_tokens"][:3].tolist() == [voc[s] for s in g["expected"]["committed"]]
    g = pins.load_golden("greedy_ties.json")
    for c in g["cases"]:
        b = synth.from_arrays(g["target_logits"], None, c["draft_tokens"], [2], greedy=[1],
                              dtype="bf16", device=DEV)
        got = run_hip(b)
        n = c["accepted_len"] + 1
        assert got["accepted_len"][0] == c["accepted_len"]
        assert got["out_tokens"][:n].tolist() == c["committed"], (c, got)


@pytest.mark.parametrize("T", [1e-20, 1e-3, 50.0, 1e6])
def test_extreme_temperatures(T):
    """Temperatures far from 1 (near-argmax and near-uniform distributions)."""
    batch = synth.make_batch(5, DEV, B=24, V=4099)
    batch.temperature = float(np.float32(T))
    got = run_hip(batch)
    ref = run_oracle(batch)
    near = compare(batch, got, ref, f"T={T}")


def test_rows_without_mass_and_huge_scaled_logits():
    """A stochastic row whose logits are all -inf has no distribution: a request
    that tests such a row reports -1, a request cut before it is verified
    normally.  Logits with |z| * log2(e)/T far above FLT_MAX (T = 1e-37, z = 100)
    are verified like any others.  All launch plans and early exit agree."""
    import draft_token_verification_row_amd as sv
    T = float(np.float32(1e-37))
    batch = synth.make_batch(3, DEV, B=6, V=1000, k=2, seed=5)
    assert np.all(batch.num_draft == 2) and np.all(batch.greedy == 0)
    batch.temperature = T
    g = torch.Generator(device="cpu").manual_seed(11)
    tgt = torch.randn(batch.target.shape, generator=g).clamp(-5, 5).to(DEV, batch.target.dtype)
    drf = torch.randn(batch.draft.shape, generator=g).clamp(-5, 5).to(DEV, batch.draft.dtype)
    toks = batch.tokens.clone()
    off = batch.offsets
    inf = float("inf")

    def trow(b, i):
        return int(off[b]) + b + i

    def drow(b, i):
        return int(off[b]) + i

    def accept_at(b, i, y):        # y is the unique maximum of both rows: p = q = 1
        tgt[trow(b, i), y] = 10.0
        drf[drow(b, i), y] = 10.0
        toks[drow(b, i)] = y

    def reject_at(b, i, y):        # y is the draft's maximum, far below the target's: p = 0
        tgt[trow(b, i), y] = -10.0
        drf[drow(b, i), y] = 10.0
        toks[drow(b, i)] = y

    reject_at(0, 0, 17)
    tgt[trow(0, 1)] = -inf         # beyond the cut: not tested
    accept_at(1, 0, 21)
    tgt[trow(1, 1)] = -inf         # tested target row without mass
    accept_at(2, 0, 22)
    drf[drow(2, 1)] = -inf         # tested draft row without mass
    tgt[trow(3, 0)] = -inf
    accept_at(4, 0, 23)
    accept_at(4, 1, 24)
    tgt[trow(4, 2)] = -inf         # the bonus row
    accept_at(5, 0, 25)
    tgt[trow(5, 1), 4] = 100.0     # |z| * log2(e)/T ~ 1.4e39
    drf[drow(5, 1), 9] = 100.0
    toks[drow(5, 1)] = 9           # p(9) = 0: rejected, the residual is one-hot at 4
    batch.target, batch.draft, batch.tokens = tgt, drf, toks
    expect_invalid = [1, 2, 3, 4]
    results = {}
    for plan in (1, 2):
        sv.spec_verify_set_launch_plan(plan)
        try:
            results[plan] = run_hip(batch)
        finally:
            sv.spec_verify_set_launch_plan(0)
    results["ee"] = run_hip(batch, max_k=2)
    good = [0, 5]
    with np.errstate(invalid="ignore"):     # request 0's all -inf row after its cut
        ref = run_oracle(synth.select_requests(batch, good, device="cpu"))
    for name, got in results.items():
        acc = got["accepted_len"]
        assert acc[expect_invalid].tolist() == [-1] * 4, (name, acc)
        for b in expect_invalid:
            assert np.all(got["out_tokens"][trow(b, 0):trow(b, 2) + 1] == -1), (name, b)
            assert np.all(got["p_draft"][drow(b, 0):drow(b, 1) + 1] == -1), (name, b)
            assert got["resid_mass"][b] == -1, (name, b)
        assert acc[good].tolist() == ref["accepted_len"].tolist() == [0, 1], (name, acc)
        for j, b in enumerate(good):
            sl = slice(trow(b, 0), trow(b, 2) + 1)
            assert got["out_tokens"][sl].tolist() == ref["out_tokens"][3 * j:3 * j + 3].tolist(), (name, b)
        assert got["out_tokens"][trow(5, 1)] == 4
    for k in ("accepted_len", "out_tokens", "resid_mass"):
        assert np.array_equal(results[1][k], results[2][k]), k
        assert np.array_equal(results[1][k], results["ee"][k]), k


def test_scale_rounding_worst_temperature():
    """T = 0.72118998 makes fl(log2(e)/T) the farthest from log2(e)/T (a relative
    5.96e-8, within 0.1 % of the 2^-24 bound over T in [0.5, 2]); with logits
    twice as wide as the workloads' the kernels' softmax at T' = log2(e)/c must
    still give p, q, Z within 1e-5 and the same decisions."""
    T = float(np.float32(0.7211899757385254))
    c64 = 1.4426950408889634 / T
    assert abs(float(np.float32(c64)) / c64 - 1.0) > 5.9e-8
    batch = synth.make_batch(5, DEV, B=48, V=30011)
    batch.temperature = T
    batch.target = (batch.target.float() * 2.0).to(batch.target.dtype)
    batch.draft = (batch.draft.float() * 2.0).to(batch.draft.dtype)
    got = run_hip(batch)
    ref = run_oracle(batch)
    near = compare(batch, got, ref, "worst scale rounding")


def test_masked_vocabulary_columns():
    batch = synth.make_batch(5, DEV, B=20, V=40000)
    batch.target[:, -3000:] = float("-inf")
    if batch.draft is not None:
        batch.draft[:, -3000:] = float("-inf")
    stoch = np.repeat(batch.greedy == 0, batch.num_draft)
    toks = batch.tokens.clone()
    bad = torch.as_tensor(stoch, device=DEV) & (toks >= 40000 - 3000)
    toks[bad] = 5
    batch.tokens = toks
    got = run_hip(batch)
    ref = run_oracle(batch)
    compare(batch, got, ref, "masked")
    out = got["out_tokens"]
    assert np.all(out[out >= 0] < 37000)


def test_repeat_calls_are_bit_identical():
    batch = synth.make_batch(5, DEV, B=64, V=30000)
    a = run_hip(batch)
    b = run_hip(batch)
    for k in a:
        if a[k] is not None:
            assert np.array_equal(a[k], b[k]), k


def test_non_default_stream():
    batch = synth.make_batch(4, DEV, B=4, V=20000)
    a = run_hip(batch)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        b = run_hip(batch, stream=s)
    s.synchronize()
    for k in a:
        if a[k] is not None:
            assert np.array_equal(a[k], b[k]), k


def test_device_side_input_errors():
    import draft_token_verification_row_amd as sv
    batch = synth.make_batch(5, DEV, B=10, V=5000)
    nd = torch.as_tensor(batch.num_draft, dtype=torch.int32, device=DEV)
    gm = torch.as_tensor(batch.greedy, dtype=torch.uint8, device=DEV)
    # sum(num_draft) != K: every output is -1
    nd_bad = nd.clone()
    nd_bad[0] += 1
    r = sv.spec_verify_sample(batch.target, batch.draft, batch.tokens, nd_bad, batch.temperature,
                              batch.u_accept, batch.u_final, greedy_mask=gm)
    torch.cuda.synchronize()
    assert torch.all(r["accepted_len"] == -1) and torch.all(r["out_tokens"] == -1)
    # a negative count is an error too
    nd_neg = nd.clone()
    nd_neg[1] = -1
    nd_neg[2] += 1
    r = sv.spec_verify_sample(batch.target, batch.draft, batch.tokens, nd_neg, batch.temperature,
                              batch.u_accept, batch.u_final, greedy_mask=gm)
    torch.cuda.synchronize()
    assert torch.all(r["accepted_len"] == -1)
    # stochastic token out of range: only that request is marked
    b0 = int(np.flatnonzero((batch.greedy == 0) & (batch.num_draft > 0))[0])
    off = batch.offsets
    toks = batch.tokens.clone()
    toks[int(off[b0])] = 5000
    r = sv.spec_verify_sample(batch.target, batch.draft, toks, nd, batch.temperature,
                              batch.u_accept, batch.u_final, greedy_mask=gm)
    torch.cuda.synchronize()
    acc = r["accepted_len"].cpu().numpy()
    assert acc[b0] == -1
    sl = slice(int(off[b0]) + b0, int(off[b0]) + b0 + int(batch.num_draft[b0]) + 1)
    assert np.all(r["out_tokens"].cpu().numpy()[sl] == -1)
    good = synth.select_requests(batch, [b for b in range(batch.B) if b != b0], device=DEV)
    ref = run_oracle(good)
    assert np.array_equal(np.delete(acc, b0), ref["accepted_len"])


def test_host_error_writes_nothing():
    import draft_token_verification_row_amd as sv
    batch = synth.make_batch(3, DEV, B=4, V=3000)
    nd = torch.as_tensor(batch.num_draft, dtype=torch.int32, device=DEV)
    acc = torch.full((batch.B,), 777, dtype=torch.int32, device=DEV)
    out = torch.full((batch.K + batch.B,), 777, dtype=torch.int32, device=DEV)
    small = torch.empty(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(sv.SpecVerifyError):
        sv.spec_verify_sample(batch.target, batch.draft, batch.tokens, nd, batch.temperature,
                              batch.u_accept, batch.u_final, accepted_len=acc, out_tokens=out,
                              workspace=small)
    with pytest.raises(sv.SpecVerifyError):
        sv.spec_verify_sample(batch.target, batch.draft, batch.tokens, nd, -1.0,
                              batch.u_accept, batch.u_final, accepted_len=acc, out_tokens=out)
    torch.cuda.synchronize()
    assert torch.all(acc == 777) and torch.all(out == 777)


def _invariants(batch, got):
    """Checks that hold for every request at any size (no oracle needed)."""
    nd = batch.num_draft.astype(np.int64)
    off = np.concatenate([[0], np.cumsum(nd)])
    acc = got["accepted_len"].astype(np.int64)
    out = got["out_tokens"].astype(np.int64)
    toks = batch.tokens.cpu().numpy().astype(np.int64)
    assert np.all((acc >= 0) & (acc <= nd))
    final_rows = []
    for b in range(batch.B):
        t0 = off[b] + b
        a = acc[b]
        assert np.array_equal(out[t0:t0 + a], toks[off[b]:off[b] + a])
        assert 0 <= out[t0 + a] < batch.V
        assert np.all(out[t0 + a + 1:t0 + nd[b] + 1] == -1)
        if a < nd[b]:
            assert out[t0 + a] != toks[off[b] + a]       # the correction never repeats the rejected draft
        final_rows.append(t0 + a)
    # greedy finals are the lowest id attaining the row maximum (checked on the device)
    g = np.flatnonzero(batch.greedy == 1)
    if g.size:
        rows = torch.as_tensor(np.array(final_rows)[g], device=DEV)
        tok = torch.as_tensor(out[np.array(final_rows)[g]], device=DEV)
        x = batch.target.index_select(0, rows).float()
        mx = x.max(dim=1).values
        assert torch.all(x.gather(1, tok[:, None])[:, 0] == mx)
        first = (x == mx[:, None]).int().argmax(dim=1)
        assert torch.equal(first, tok)
        # and every kept greedy draft attains its row maximum
        for b in g[:64]:
            for i in range(acc[b]):
                row = batch.target[off[b] + b + i].float()
                assert row[toks[off[b] + i]] == row.max()


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_full_size_every_request(cfg):
    """Each workload at its real shape, in the launch configuration the
    benchmark times: every request against the oracle, plus the invariants."""
    _log(f"[full] cfg={cfg} generating")
    batch = synth.make_batch(cfg, DEV)
    torch.cuda.synchronize()
    _log(f"[full] cfg={cfg} B={batch.B} K={batch.K} V={batch.V} running")
    got = run_hip(batch)
    _invariants(batch, got)
    _log(f"[full] cfg={cfg} oracle on all {batch.B} requests")
    ref = run_oracle(batch, chunk=32)
    near = compare(batch, got, ref, f"full cfg{cfg}")
    _log(f"[full] cfg={cfg}: {batch.B} requests, near_ties={near}, "
         f"mean accepted={got['accepted_len'].mean():.3f}")


def test_monte_carlo_distribution_on_gpu():
    """One batch of 10^6 requests over the same small rows, fresh drafts y ~ q and
    fresh uniforms: committed-token and accepted-length frequencies match the
    closed forms of the method's guarantee (every cell within 5 sigma)."""
    import scipy.special
    rng = np.random.default_rng(2024)
    V, k, N, T = 8, 3, 1000000, 0.9
    z = rng.normal(0, 1.5, size=(k + 1, V))
    d = z[:k] + rng.normal(0, 1.0, size=(k, V))
    z32, d32 = z.astype(np.float32), d.astype(np.float32)
    Tf = float(np.float32(T))
    P = [scipy.special.softmax(z32[i].astype(np.float64) / Tf) for i in range(k + 1)]
    Q = [scipy.special.softmax(d32[i].astype(np.float64) / Tf) for i in range(k)]
    beta = [float(np.minimum(P[i], Q[i]).sum()) for i in range(k)]
    ys = np.stack([np.minimum(np.searchsorted(np.cumsum(Q[i]), rng.random(N), side="right"), V - 1)
                   for i in range(k)], axis=1)
    target = torch.as_tensor(np.tile(z32, (N, 1)), device=DEV)
    draft = torch.as_tensor(np.tile(d32, (N, 1)), device=DEV)
    batch = synth.Batch(
        name="mc", B=N, K=N * k, V=V, dtype="f32", num_draft=np.full(N, k, np.int32),
        greedy=np.zeros(N, np.uint8), temperature=Tf, target=target, draft=draft,
        tokens=torch.as_tensor(ys.reshape(-1).astype(np.int32), device=DEV),
        u_accept=torch.as_tensor(synth.uniforms_f32(rng, N * k), device=DEV),
        u_final=torch.as_tensor(synth.uniforms_f32(rng, N), device=DEV))
    got = run_hip(batch, want_probs=False)
    A = got["accepted_len"].astype(np.int64)
    out = got["out_tokens"].reshape(N, k + 1)

    def close(count, n, prob):
        return abs(count - n * prob) <= 5.0 * math.sqrt(n * prob * (1 - prob)) + 1.0

    first = np.bincount(out[:, 0], minlength=V)
    assert all(close(first[v], N, P[0][v]) for v in range(V)), (first / N, P[0])
    for j in range(1, k + 1):
        surv = float(np.prod(beta[:j]))
        assert close(int((A >= j).sum()), N, surv), (j, (A >= j).mean(), surv)
        reached = A >= j
        cnt = np.bincount(out[reached, j], minlength=V)
        assert all(close(cnt[v], int(reached.sum()), P[j][v]) for v in range(V)), (j, cnt)
    prog = oracle.expected_progress(beta, k)
    assert abs(A.mean() + 1 - prog) <= 5 * math.sqrt(A.var() / N)
