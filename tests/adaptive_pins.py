"""Pins of the adaptive-length oracle (chzhyang, "Speculative Decoding: ...",
section 5 DSpark and section 2), to facts that do not come from the oracle:

* progress(k) in closed form for constant confidence (geometric series), and
  as 1 + E[A] computed by enumerating the distribution of the accepted length
  A that the survival estimates s_j describe;
* special cases whose choice is fixed by monotonicity (costs flat, costs
  growing faster or slower than progress, a zero confidence), and ties;
* brute force: the choice minimises the time per token cost[k] / progress(k)
  of section 2 (vectorised, a different arithmetic route) on random inputs;
* a hand-derived compaction of three requests into the packed layout.
Every pin calls the oracle through its module.
"""
import numpy as np

import oracle.adaptive as oa


def pin_progress_closed_form():
    for c0 in (0.0, 0.25, 0.5, 0.875, 1.0):
        conf = np.full(9, c0, np.float32)
        prog = oa.progress_table(conf)
        for k in range(10):
            want = k + 1.0 if c0 == 1.0 else (1.0 - c0 ** (k + 1)) / (1.0 - c0)
            assert abs(prog[k] - want) <= 1e-14 * want, (c0, k, prog[k], want)
    rng = np.random.default_rng(21)
    for _ in range(200):
        n = int(rng.integers(0, 9))
        conf = rng.random(n).astype(np.float32)
        prog = oa.progress_table(conf)
        for k in range(n + 1):
            # P(A = j) = s_j (1 - c_{j+1}) for j < k, P(A = k) = s_k
            s = [1.0]
            for j in range(k):
                s.append(s[-1] * float(conf[j]))
            pa = [s[j] * (1.0 - float(conf[j])) for j in range(k)] + [s[k]]
            ea = sum(j * p for j, p in enumerate(pa))
            assert abs(sum(pa) - 1.0) < 1e-12
            assert abs(prog[k] - (1.0 + ea)) < 1e-12, (conf, k)


def pin_choice_special_cases():
    N = 7
    conf = np.full(N, 0.8, np.float32)
    assert oa.choose_length(conf, np.ones(N + 1))[0] == N          # flat cost: all positions
    flat = np.ones(N, np.float32)
    for m, want in ((0.5, N), (2.0, 0), (1.0, 0)):                 # progress 1+k vs cost 1+mk
        cost = 1.0 + m * np.arange(N + 1)
        assert oa.choose_length(flat, cost)[0] == want, m
    z = np.array([0.0] + [0.9] * (N - 1), np.float32)               # s_j = 0 for all j: tie
    assert oa.choose_length(z, np.ones(N + 1)) == (0, 1.0)
    mid = np.array([0.9, 0.9, 0.0, 0.9, 0.9, 0.9, 0.9], np.float32)  # progress flat from k = 2
    k, p = oa.choose_length(mid, np.ones(N + 1))
    assert k == 2 and abs(p - (1 + 0.9 + 0.81)) < 1e-6
    # cost grows by 0.15 per position: stop once the next survival is worth less
    cost = 1.0 + 0.15 * np.arange(N + 1)
    conf = np.array([0.95, 0.9, 0.6, 0.3, 0.2, 0.1, 0.05], np.float32)
    k, _ = oa.choose_length(conf, cost)
    prog = np.cumsum(np.concatenate([[1.0], np.cumprod(conf.astype(np.float64))]))
    assert k == int(np.argmax(prog / cost)) and 0 < k < N
    # the worked numbers of section 2: 18 ms per round over progress 4 and 2
    assert abs(18.0 / oa.progress_table(np.ones(3, np.float32))[3] - 4.5) < 1e-12
    assert abs(18.0 / oa.progress_table(np.array([1.0, 0.0, 0.0], np.float32))[3] - 9.0) < 1e-12


def pin_brute_force_time_per_token():
    rng = np.random.default_rng(22)
    for _ in range(500):
        N = int(rng.integers(1, 16))
        conf = rng.random(N).astype(np.float32)
        cost = 1.0 + np.cumsum(rng.random(N + 1)) * rng.random()
        surv = np.cumprod(conf.astype(np.float64))
        prog = 1.0 + np.concatenate([[0.0], np.cumsum(surv)])
        tpt = cost / prog
        want = int(np.flatnonzero(tpt == tpt.min())[0])
        k, p = oa.choose_length(conf, cost)
        if k != want:   # only an exact tie in the other direction's rounding may differ
            r = prog / cost
            assert abs(r[k] - r[want]) <= 1e-15 * r[want], (conf, cost, k, want)
        assert abs(p - prog[k]) <= 1e-14 * prog[k]


def pin_compaction():
    N = 4
    conf = np.array([[0.9, 0.9, 0.0, 0.5], [0.0, 0.9, 0.9, 0.9], [0.9, 0.9, 0.9, 0.9]], np.float32)
    tokens = np.array([[11, 12, 13, 14], [21, 22, 23, 24], [31, 32, 33, 34]])
    r = oa.adaptive_batch(conf, np.ones(N + 1), tokens)
    assert r["num_draft"].tolist() == [2, 0, 4]
    assert r["offsets"].tolist() == [0, 2, 2, 6]
    assert r["src_index"].tolist() == [0, 1, 8, 9, 10, 11]
    assert r["tokens"].tolist() == [11, 12, 31, 32, 33, 34]
    assert np.allclose(r["progress"], [1.0 + 0.9 + 0.81, 1.0, 1 + 0.9 + 0.81 + 0.729 + 0.6561], rtol=1e-6)
    for bad in (np.ones(N), np.array([1.0, 1.0, 0.0, 1.0, 1.0])):
        try:
            oa.adaptive_batch(conf, bad, tokens)
        except ValueError:
            continue
        raise AssertionError("invalid cost table accepted")


ADAPTIVE_PINS = [pin_progress_closed_form, pin_choice_special_cases, pin_brute_force_time_per_token,
                 pin_compaction]
