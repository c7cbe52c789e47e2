"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each pin is a plain function taking the oracle's `verify` module, so the same
checks run on the oracle as written (tests/test_oracle_pins.py) and on copies
with a planted mistake (tests/test_oracle_mutants.py), which must fail at least
one pin.  Nothing here retypes the oracle's formulas: expectations come from
the pages' worked examples, hand-derived closed forms, scipy / numpy routines
the oracle does not call, and exact statistics of the construction.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import scipy.special

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_golden(name: str) -> dict:
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _logits_from_probs(rows) -> np.ndarray:
    p = np.asarray(rows, dtype=np.float64)
    out = np.full(p.shape, -1000.0)
    pos = p > 0
    out[pos] = np.log(p[pos])
    return out


def _run(vm, target, draft, tokens, greedy, T, u, w):
    return vm.verify_request(np.asarray(target, np.float64),
                             None if draft is None else np.asarray(draft, np.float64),
                             np.asarray(tokens), greedy, T, np.asarray(u, np.float64), w)


# ---------------------------------------------------------------- worked examples
def pin_abr_example(vm):
    """A B C D -> A B R for every uniform that rejects C ([CZ] section 1)."""
    g = load_golden("abr_example.json")
    voc = {s: i for i, s in enumerate(g["vocab"])}
    tgt = _logits_from_probs(g["target_probs"])
    dr = _logits_from_probs(g["draft_probs"])
    toks = [voc[s] for s in g["draft_tokens"]]
    thr = g["reject_threshold_C"]
    grid = [0.0, 0.1, 0.37, 0.5, 0.8, 0.999]
    for uA in grid:
        for uC in [thr + 1e-6, 0.3, 0.6, 0.99]:
            for w in [0.0, 0.2, 0.5, 0.9, 0.9999]:
                r = _run(vm, tgt, dr, toks, False, g["temperature"], [uA, 1.0 - uA, uC, 0.0], w)
                assert r["a"] == g["expected"]["accepted_len"], (uA, uC, w, r)
                assert r["committed"] == [voc[s] for s in g["expected"]["committed"]], (uA, uC, w, r)
    # a uniform below p/q keeps C, so the round goes on past position 2
    r = _run(vm, tgt, dr, toks, False, 1.0, [0.5, 0.5, thr - 1e-6, 0.99], 0.5)
    assert r["a"] >= 3 and r["committed"][:3] == toks[:3], r
    # k = 2: both drafts survive and the bonus comes from target row 2 by inverse CDF
    tk = g["truncated_k2_expected"]
    for w, name in tk["bonus_for_w"]:
        r = _run(vm, tgt[:3], dr[:2], toks[:2], False, 1.0, [0.9, 0.9], w)
        assert r["a"] == tk["accepted_len"], r
        assert r["committed"] == toks[:2] + [voc[name]], (w, r)


def pin_weather_example(vm):
    """Greedy: sunny and warm outside -> sunny and clear ([VLLM] accept/reject example)."""
    g = load_golden("weather_example.json")
    voc = {s: i for i, s in enumerate(g["vocab"])}
    toks = [voc[s] for s in g["draft_tokens"]]
    r = _run(vm, g["target_logits"], None, toks, True, None, [0.0] * 4, 0.0)
    assert r["a"] == g["expected"]["accepted_len"], r
    assert r["committed"] == [voc[s] for s in g["expected"]["committed"]], r


def pin_t1_t4_round(vm):
    """T1 T2 T3 T4, check check cross: commit T1 T2 + replacement from [p-q]_+ ([HN], [CZ] s.1)."""
    g = load_golden("round_t1_t4.json")
    voc = {s: i for i, s in enumerate(g["vocab"])}
    tgt = _logits_from_probs(g["target_probs"])
    dr = _logits_from_probs(g["draft_probs"])
    toks = [voc[s] for s in g["draft_tokens"]]
    for uC in [0.2 + 1e-6, 0.5, 0.95]:
        for w, name in g["expected"]["replacement_for_w"]:
            r = _run(vm, tgt, dr, toks, False, 1.0, [0.99, 0.99, uC, 0.0], w)
            assert r["a"] == g["expected"]["accepted_len"], r
            assert r["committed"] == [voc[s] for s in g["expected"]["committed_prefix"]] + [voc[name]], (uC, w, r)


def pin_greedy_ties(vm):
    """Lowest id wins a tied maximum (the library's reading of greedy equivalence)."""
    g = load_golden("greedy_ties.json")
    for c in g["cases"]:
        r = _run(vm, g["target_logits"], None, c["draft_tokens"], True, None, [0.0, 0.0], 0.0)
        assert r["a"] == c["accepted_len"] and r["committed"] == c["committed"], (c, r)


# ---------------------------------------------------------------- closed forms
def _rows(rng, V, k, sigma=1.5, noise=1.0):
    z = rng.normal(0.0, sigma, size=(k + 1, V))
    d = z[:k] + rng.normal(0.0, noise, size=(k, V))
    return z, d


def pin_exact_distribution_quadrature(vm, G: int = 1024):
    """V = 3, k = 1: with y ~ q enumerated exactly and (u, w) swept over a 1/G grid of
    midpoints, the committed token's frequency equals p (the target-distribution
    guarantee of [CZ] section 1) within the grid resolution; k = 0 gives p too."""
    rng = np.random.default_rng(7)
    grid = (np.arange(G) + 0.5) / G
    for T in (1.0, 0.7):
        z, d = _rows(rng, 3, 1)
        p = scipy.special.softmax(z[0] / np.float32(T))
        q = scipy.special.softmax(d[0] / np.float32(T))
        # acceptance frequency for each possible draft, from the u sweep
        acc = np.zeros(3)
        for y in range(3):
            acc[y] = np.mean([_run(vm, z, d, [y], False, T, [u], 0.5)["a"] == 1 for u in grid])
            assert abs(acc[y] - min(1.0, p[y] / q[y])) <= 1.0 / G + 1e-12, (y, acc[y], p[y] / q[y])
        # correction distribution, from the w sweep with a rejecting uniform
        y_rej = int(np.argmin(p / q))
        corr = np.zeros(3)
        for w in grid:
            r = _run(vm, z, d, [y_rej], False, T, [0.999999], w)
            assert r["a"] == 0
            corr[r["committed"][0]] += 1.0 / G
        freq = np.zeros(3)
        for y in range(3):
            freq[y] += q[y] * acc[y]
            freq += q[y] * (1.0 - acc[y]) * corr
        assert np.all(np.abs(freq - p) <= 3.0 / G), (freq, p)
        # k = 0: the bonus alone is a draw from p
        bon = np.zeros(3)
        for w in grid:
            bon[_run(vm, z[1:], d[:0], [], False, T, [], w)["committed"][0]] += 1.0 / G
        pb = scipy.special.softmax(z[1] / np.float32(T))
        assert np.all(np.abs(bon - pb) <= 1.0 / G + 1e-12), (bon, pb)


def pin_monte_carlo(vm, trials: int = 12000, cases=((2, 1), (3, 3), (8, 1), (16, 3)), seed=11):
    """Monte Carlo against the closed forms of [CZ] sections 1 and 5:
    * the first committed token and the token at position j (given position j is
      reached) are distributed as p_j;
    * P(A >= j) = prod_{i<j} beta_i with beta_i = sum_v min(p_i, q_i);
    * E[A] + 1 equals DSpark's progress 1 + sum_j s_j with c_i = beta_i.
    Every cell must lie within 5 sigma of its expectation."""
    from oracle.cost_model import expected_progress
    rng = np.random.default_rng(seed)
    T = 0.9
    for V, k in cases:
        z, d = _rows(rng, V, k)
        P = [scipy.special.softmax(z[i] / np.float32(T)) for i in range(k + 1)]
        Q = [scipy.special.softmax(d[i] / np.float32(T)) for i in range(k)]
        beta = [float(np.minimum(P[i], Q[i]).sum()) for i in range(k)]
        A = np.zeros(trials, np.int64)
        first = np.zeros(V)
        at_pos = [np.zeros(V) for _ in range(k + 1)]
        for n in range(trials):
            ys = [int(rng.choice(V, p=Q[i])) for i in range(k)]
            u = rng.random(k)
            w = rng.random()
            r = _run(vm, z, d, ys, False, T, u, w)
            A[n] = r["a"]
            first[r["committed"][0]] += 1
            for j, t in enumerate(r["committed"]):
                at_pos[j][t] += 1
        def close(count, n, prob):
            return abs(count - n * prob) <= 5.0 * math.sqrt(n * prob * (1 - prob)) + 1.0
        assert all(close(first[v], trials, P[0][v]) for v in range(V)), (V, k, first / trials, P[0])
        for j in range(1, k + 1):
            surv = float(np.prod(beta[:j]))
            assert close(int((A >= j).sum()), trials, surv), (V, k, j, (A >= j).mean(), surv)
            reached = int((A >= j).sum())
            if reached > 200:
                assert all(close(at_pos[j][v], reached, P[j][v]) for v in range(V)), (V, k, j)
        mean_prog = expected_progress(beta, k)
        sd = math.sqrt(max(np.var(A), 1e-12) / trials)
        assert abs(A.mean() + 1.0 - mean_prog) <= 5.0 * sd + 1e-9, (A.mean() + 1, mean_prog)


# ---------------------------------------------------------------- special cases
def pin_special_cases(vm):
    rng = np.random.default_rng(3)
    V = 40
    z, d = _rows(rng, V, 3)
    T = 0.8
    # softmax equals scipy's at the fp32-widened temperature
    for TT in (0.25, 0.7, 1.0, 1.9):
        ref = scipy.special.softmax(z[0] / float(np.float32(TT)))
        got = vm.tempered_softmax(z[0], vm.widen_temperature(TT))
        assert np.allclose(got, ref, rtol=1e-13, atol=0), TT
    # k = 0: the bonus is inverse-CDF sampling of p (numpy searchsorted, side='right')
    p = scipy.special.softmax(z[0] / np.float32(T))
    F = np.cumsum(p)
    for w in np.linspace(0.0, 0.999, 97):
        if np.min(np.abs(F - w)) < 1e-9:
            continue
        want = int(np.searchsorted(F, w, side="right"))
        got = _run(vm, z[:1], d[:0], [], False, T, [], float(w))["committed"][0]
        assert got == want, (w, got, want)
    # q == p: every draft survives for any u < 1, then a bonus from the last row
    y = [3, 7, 11]
    r = _run(vm, z, z[:3].copy(), y, False, T, [0.999999, 0.999999, 0.999999], 0.3)
    assert r["a"] == 3 and r["committed"][:3] == y, r
    # q one-hot at y: y survives iff u < p(y); the correction is p with y removed
    onehot = np.full((1, V), -1000.0)
    onehot[0, 5] = 0.0
    p0 = scipy.special.softmax(z[0] / np.float32(T))
    for u in (0.5 * p0[5], 1.5 * p0[5], 0.9):
        r = _run(vm, z[:2], onehot, [5], False, T, [u], 0.4)
        assert (r["a"] == 1) == (u < p0[5]), (u, p0[5], r)
    rest = p0.copy()
    rest[5] = 0.0
    Fr = np.cumsum(rest / rest.sum())
    for w in np.linspace(0.001, 0.999, 53):
        if np.min(np.abs(Fr - w)) < 1e-9:
            continue
        got = _run(vm, z[:2], onehot, [5], False, T, [0.999999], float(w))["committed"]
        assert got == [int(np.searchsorted(Fr, w, side="right"))], (w, got)
    # p(y) = 0 (token masked in the target): rejected even with u = 0
    zm = z[:2].copy()
    zm[0, 9] = -np.inf
    r = _run(vm, zm, d[:1], [9], False, T, [0.0], 0.5)
    assert r["a"] == 0 and r["committed"][0] != 9, r
    # masked ids are never committed; zero-weight ids are never drawn, even at w = 0
    zm = z.copy()
    zm[:, :4] = -np.inf
    for w in (0.0, 1e-9, 0.5):
        r = _run(vm, zm[3:], d[:0], [], False, T, [], w)
        assert r["committed"][0] >= 4, (w, r)
    # a tiny temperature turns the bonus draw into the row argmax
    zz = z[3].copy()
    top = int(np.flatnonzero(zz == zz.max())[0])
    zz[top] += 0.1                      # top gap >= 0.1: p(top) > 1 - 1e-40 at T = 1e-3
    for w in (0.01, 0.5, 0.99):
        r = _run(vm, zz[None, :], d[:0], [], False, 1e-3, [], w)
        assert r["committed"] == [top], r
    # the temperature matters: at T = 0.25 vs T = 4 the bonus differs for some w
    outs = set()
    for TT in (0.25, 4.0):
        outs.add(tuple(_run(vm, z[:1], d[:0], [], False, TT, [], w)["committed"][0]
                       for w in (0.1, 0.3, 0.5, 0.7, 0.9)))
    assert len(outs) == 2


def pin_temperature_reading(vm):
    """Reading R1: the kernels take the temperature as an fp32 value, so an
    fp64 T given to the oracle acts as fp32(T): p(y) and q(y) equal scipy's
    softmax of z / fp32(T), which differs measurably from z / T here."""
    rng = np.random.default_rng(8)
    V = 50
    z, d = _rows(rng, V, 2, sigma=3.0)
    for T in (0.7, 0.3, 1.3):
        T32 = float(np.float32(T))
        r = _run(vm, z, d, [3, 5], False, T, [0.999999, 0.999999], 0.5)
        for i, y in ((0, 3),):
            want_p = scipy.special.softmax(z[i] / T32)[y]
            want_q = scipy.special.softmax(d[i] / T32)[y]
            other = scipy.special.softmax(z[i] / T)[y]
            assert abs(want_p - other) > 1e-11 * want_p, T      # the two readings differ
            assert abs(r["p_y"][i] - want_p) <= 1e-13 * want_p, (T, r["p_y"][i], want_p)
            assert abs(r["q_y"][i] - want_q) <= 1e-13 * want_q, (T, r["q_y"][i], want_q)


def pin_greedy_invariants(vm, n_req: int = 300, V: int = 64, k: int = 4, seed: int = 5):
    """On random rows with many exact ties: every kept draft attains its row's
    maximum and no lower id does; the token at the cut attains the maximum with
    no lower id doing so; a cut before k means the draft there was not that token."""
    rng = np.random.default_rng(seed)
    for _ in range(n_req):
        z = np.round(rng.normal(0, 1.0, size=(k + 1, V)) * 4) / 4   # coarse grid -> ties
        m = z.max(axis=1)
        ys = []
        for i in range(k):
            ids = np.flatnonzero(z[i] == m[i])
            ys.append(int(ids[0]) if rng.random() < 0.6 else int(rng.integers(0, V)))
        r = _run(vm, z, None, ys, True, None, [0.0] * k, 0.0)
        a, c = r["a"], r["committed"]
        assert len(c) == a + 1 and c[:a] == ys[:a]
        for i in range(a + 1):
            t = c[i]
            assert z[i, t] == m[i] and not np.any(z[i, :t] == m[i]), (i, t)
        if a < k:
            assert ys[a] != c[a]


def pin_cost_model():
    """[CZ] section 2 illustration: 3 + 13 + 2 ms per round; A = 3 -> 4.5 ms/token,
    A = 1 -> 9 ms/token, both below the 10 ms/token of ordinary decoding."""
    from oracle.cost_model import time_per_token, expected_progress
    assert time_per_token(3.0, 13.0, 2.0, 3.0) == 4.5
    assert time_per_token(3.0, 13.0, 2.0, 1.0) == 9.0
    assert time_per_token(3.0, 13.0, 2.0, 0.0) == 18.0
    assert expected_progress([1.0, 1.0, 1.0], 3) == 4.0
    assert expected_progress([0.5, 0.5], 2) == 1.75
    assert expected_progress([0.9, 0.5, 0.2], 0) == 1.0


def pin_packed_batch(vm):
    """Ragged packing: requests of different k placed back to back give each
    request's own fixture answer (offsets off[b] + b + i / off[b] + i)."""
    g = load_golden("abr_example.json")
    voc = {s: i for i, s in enumerate(g["vocab"])}
    tgt = _logits_from_probs(g["target_probs"])
    dr = _logits_from_probs(g["draft_probs"])
    toks = [voc[s] for s in g["draft_tokens"]]
    ks = [3, 0, 2, 4]
    T_rows, D_rows, Y, U, W = [], [], [], [], []
    for kk in ks:
        T_rows.extend(tgt[:kk + 1])
        D_rows.extend(dr[:kk])
        Y.extend(toks[:kk])
        U.extend([0.9, 0.9, 0.5, 0.1][:kk])
        W.append(0.5)
    res = vm.verify_batch(np.array(T_rows), np.array(D_rows).reshape(-1, 6), np.array(Y),
                          np.array(ks), np.zeros(4, bool), 1.0, np.array(U, np.float32),
                          np.array(W, np.float32))
    R, A = voc["R"], voc["A"]
    # k=3 (A B C, u_C = 0.5 >= 1/6 rejects) -> A B R;  k=0 -> bonus from p0 at w=.5
    # (cumulative .40 .55 -> B);  k=2 -> A B + bonus from p2 at w=.5 (-> R);  k=4 -> A B R
    assert list(res["accepted_len"]) == [2, 0, 2, 2], res["accepted_len"]
    off = np.concatenate([[0], np.cumsum(ks)])
    got = [list(res["out_tokens"][off[b] + b: off[b] + b + ks[b] + 1]) for b in range(4)]
    assert got[0] == [A, voc["B"], R, -1], got
    assert got[1] == [voc["B"]], got
    assert got[2] == [A, voc["B"], R], got
    assert got[3] == [A, voc["B"], R, -1, -1], got
    assert np.all(res["resid_mass"][[0, 3]] > 0) and res["resid_mass"][1] == -1.0


# ---------------------------------------------------------------- decision margins
def pin_decision_margins(vm):
    """The margins that decide which GPU/oracle disagreements count as
    near-ties, against hand-derived values.

    Ratio test: |u q - p| / max(u q, p).  Draw: distance of w * total from the
    nearer edge of the chosen token's cumulative interval, relative to the
    total.  A request's margin is the smallest over the ratio tests up to and
    including its cut plus the final draw (later positions decide nothing)."""
    am = vm.accept_margin
    for (u, p, q), want in (((0.5, 0.1, 0.4), 0.5),         # 0.2 vs 0.1
                            ((0.25, 0.1, 0.4), 0.0),        # 0.1 vs 0.1 exactly
                            ((0.9, 0.3, 0.3), 0.1),         # 0.27 vs 0.3
                            ((0.5, 0.3, 0.1), 0.25 / 0.3),  # 0.05 vs 0.3
                            ((0.5, 1e-13, 4e-13), 0.5),     # scale free
                            ((0.5, 0.0, 0.0), 1.0)):        # 0 vs 0: decided exactly
        got = am(u, p, q)
        assert abs(got - want) <= 1e-12, ((u, p, q), got, want)
    # weights 1 2 3 4: cumulative 1 3 6 10, total 10
    W = np.array([1.0, 2.0, 3.0, 4.0])
    for w, tok, want in ((0.375, 2, 0.075),     # 3.75 in [3, 6): lower edge nearer
                         (0.5625, 2, 0.0375),   # 5.625 in [3, 6): upper edge nearer
                         (0.25, 1, 0.05),       # 2.5 in [1, 3)
                         (0.0, 0, 0.0),         # 0 on the lower edge of token 0
                         (0.95, 3, 0.05)):      # 9.5 in [6, 10)
        for scale in (1.0, 2.0 ** -30, 2.0 ** 20):     # relative to the total
            t, total, m = vm.inverse_cdf(W * scale, w)
            assert t == tok and abs(total - 10.0 * scale) <= 1e-12 * scale, (w, scale, t, total)
            assert abs(m - want) <= 1e-12, (w, scale, m, want)
    # zero-weight ids: cumulative 0 2 2 4
    t, _, m = vm.inverse_cdf(np.array([0.0, 2.0, 0.0, 2.0]), 0.25)
    assert t == 1 and abs(m - 0.25) <= 1e-12, (t, m)
    t, _, m = vm.inverse_cdf(np.array([0.0, 2.0, 0.0, 2.0]), 0.5)
    assert t == 3 and m == 0.0, (t, m)
    # request: p0 = .1 .2 .3 .4, q0 = .4 .3 .2 .1, y0 = 0, u0 = .5 -> reject
    # (margin .5); residual 0 0 .1 .3 (Z = .4), w = .5 -> 0.2 in [.1, .4)
    # -> token 3, margin min(.1, .2)/.4 = .25.  Position 1 (after the cut) has
    # a test 0.0099 from its boundary that decides nothing.
    tgt = _logits_from_probs([[0.1, 0.2, 0.3, 0.4], [0.25] * 4, [0.7, 0.1, 0.1, 0.1]])
    dr = _logits_from_probs([[0.4, 0.3, 0.2, 0.1], [0.5, 0.2, 0.2, 0.1]])
    r = _run(vm, tgt, dr, [0, 0], False, 1.0, [0.5, 0.505], 0.5)
    assert r["a"] == 0 and r["committed"] == [3], r
    assert abs(r["resid_mass"] - 0.4) <= 1e-12, r
    assert abs(r["margin"] - 0.25) <= 1e-9, r["margin"]
    # u0 = .9: reject with margin |.36 - .1| / .36; the draw margin (.25) is smaller
    r = _run(vm, tgt, dr, [0, 0], False, 1.0, [0.9, 0.505], 0.5)
    assert r["a"] == 0 and abs(r["margin"] - 0.25) <= 1e-9, r
    # u0 = .2: reject on the boundary itself (.08 vs .1 keeps: .2 * .4 = .08 < .1)
    # -> kept; u1 = .505 rejects position 1 (.2525 vs .25, margin .0099)
    r = _run(vm, tgt, dr, [0, 0], False, 1.0, [0.2, 0.505], 0.5)
    assert r["a"] == 1, r
    assert abs(r["margin"] - (0.2525 - 0.25) / 0.2525) <= 1e-9, r["margin"]
    # greedy requests have no margin
    assert math.isinf(_run(vm, tgt, None, [3, 0], True, None, [0, 0], 0.5)["margin"])


def pin_early_exit_form(vm, n_batches: int = 6, seed: int = 31):
    """The left-to-right form that computes a position's distributions only
    when its test is reached gives the same decisions, tokens, residual masses
    and margins as the form that computes every row, and p(y), q(y) at the
    tested positions (-1 after the cut)."""
    rng = np.random.default_rng(seed)
    for _ in range(n_batches):
        B, V = 12, int(rng.integers(2, 60))
        ks = rng.integers(0, 6, size=B)
        K = int(ks.sum())
        off = np.concatenate([[0], np.cumsum(ks)])
        tgt = rng.normal(0, 2.0, size=(K + B, V))
        dr = np.zeros((K, V))
        for b in range(B):
            for i in range(int(ks[b])):      # draft row (b, i) = target row (b, i) + noise
                dr[off[b] + i] = tgt[off[b] + b + i] + rng.normal(0, 0.7, size=V)
        toks = rng.integers(0, V, size=K)
        greedy = rng.random(B) < 0.3
        u, wf = rng.random(K), rng.random(B)
        full = vm.verify_batch(tgt, dr, toks, ks, greedy, 0.9, u, wf)
        ee = vm.verify_batch(tgt, dr, toks, ks, greedy, 0.9, u, wf, early_exit=True)
        for key in ("accepted_len", "out_tokens", "resid_mass", "margin"):
            assert np.array_equal(full[key], ee[key]), key
        for b in range(B):
            if greedy[b]:
                continue
            n = min(int(full["accepted_len"][b]) + 1, int(ks[b]))
            s0 = slice(int(off[b]), int(off[b]) + n)
            s1 = slice(int(off[b]) + n, int(off[b + 1]))
            for key in ("p_draft", "q_draft"):
                assert np.array_equal(ee[key][s0], full[key][s0])
                assert np.all(ee[key][s1] == -1.0) and np.all(full[key][s1] >= 0.0)


ALL_PINS = [pin_abr_example, pin_weather_example, pin_t1_t4_round, pin_greedy_ties,
            pin_exact_distribution_quadrature, pin_special_cases, pin_greedy_invariants,
            pin_packed_batch, pin_decision_margins, pin_early_exit_form,
            pin_temperature_reading]


# ---------------------------------------------------------------- acceptance statistics
def pin_acceptance_appendix(am, B: int = 20000):
    """All 356 rows of the [VLLM] Appendix tables in the fixture: rounds built so that
    #{A >= j} / B equals each printed p_j reproduce the printed MAL and AR
    (MAL counts the final token, AR = (MAL - 1) / N), within the rounding of
    the printing: p_j whole percent (so MAL within N * 0.005 + 0.005) and AR
    one decimal percent (within 0.5 + 0.05 points)."""
    g = load_golden("appendix_acceptance_all.json")
    assert len(g["rows"]) == 356
    for r in g["rows"]:
        N = r["N"]
        c = [int(round(p / 100.0 * B)) for p in r["p"]] + [0]
        acc = []
        acc += [0] * (B - c[0])
        for j in range(1, N + 1):
            acc += [j] * (c[j - 1] - c[j])
        st = am.acceptance_stats(np.array(acc), np.full(B, N), N)
        assert st["rounds"] == B
        assert np.allclose(st["per_position"], np.array(r["p"]) / 100.0, atol=1.0 / B), (r, st)
        assert abs(st["mal"] - r["MAL"]) <= N * 0.005 + 0.005 + 1e-9, (r["table"], N, st["mal"], r["MAL"])
        assert abs(100.0 * st["ar"] - r["AR"]) <= 0.55 + 1e-9, (r["table"], N, st["ar"], r["AR"])
        assert abs(st["ar"] - (st["mal"] - 1.0) / N) < 1e-12


def pin_acceptance_ragged(am):
    """Hand-derived ragged case: per-position denominators count only rounds that
    proposed position j; invalid rounds (accepted length -1) are ignored."""
    st = am.acceptance_stats(np.array([2, 1, 0, 0, -1]), np.array([3, 1, 0, 2, 5]), 4)
    assert st["rounds"] == 4
    assert st["mean_accepted"] == 0.75 and st["mal"] == 1.75 and st["ar"] == 0.5
    assert np.allclose(st["per_position"], [2 / 3, 1 / 2, 0.0, -1.0], rtol=0, atol=1e-15)


ACCEPT_PINS = [pin_acceptance_appendix, pin_acceptance_ragged]
