"""Host-side pieces of bench.py (no GPU): the one-GPU guard and the accounting
of the rows an early-exit call streams."""
import os
import subprocess
import sys

import numpy as np

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "GPU" in (r.stdout + r.stderr)


def test_early_exit_windows_double():
    for max_k in range(0, 300):
        wins = bench.early_exit_windows(max_k)
        assert wins[0] == (0, 1)
        assert wins[-1][1] == max_k + 1
        for (lo, hi), (lo2, _) in zip(wins, wins[1:]):
            assert hi == lo2 and hi > lo
        for r, (lo, hi) in enumerate(wins[:-1]):
            assert hi == (1 << r)          # windows end at 1, 2, 4, 8, ...
        assert len(wins) == (1 if max_k == 0 else max_k.bit_length() + 1)


def test_early_exit_rows_between_exact_and_twice_exact():
    rng = np.random.default_rng(3)
    for _ in range(200):
        B = int(rng.integers(1, 40))
        k = rng.integers(0, 40, size=B)
        acc = np.array([int(rng.integers(0, kk + 1)) for kk in k])
        st = rng.random(B) < 0.5
        max_k = int(k.max()) + int(rng.integers(0, 5))
        got = bench.early_exit_rows_read(acc, k, st, max_k)
        exact = int((acc + 1).sum() + np.minimum(acc + 1, k)[st].sum())
        full = int((k + 1).sum() + k[st].sum())
        assert exact <= got <= min(full, 2 * exact)


def test_c_oracle_baseline_helpers():
    """The C oracle timing leg of the CPU baseline: both forms, one and several
    threads, and its agreement with the NumPy oracle on the same batch."""
    import synth
    b = synth.make_batch(5, "cpu", B=20, V=3001)
    res, times = bench.run_c_oracle_timed(b, 3)
    assert set(times) == {("all_rows", 1), ("all_rows", 3), ("early_exit", 1), ("early_exit", 3)}
    assert all(t > 0 for t in times.values())
    ref, _ = bench.run_oracle_timed(bench.oracle_inputs(b), 2, False)
    assert bench.oracles_agree(b, res, ref)
    bad = dict(res, out_tokens=res["out_tokens"].copy())
    bad["out_tokens"][0] += 1
    assert not bench.oracles_agree(b, bad, ref)


def test_parity_summary_classifies_requests():
    """The bench's parity field: equal requests pass, a stochastic request that
    differs with the oracle's deciding margin below 1e-6 is a near-tie, any
    other difference (or any greedy difference) is a mismatch."""
    import synth
    b = synth.make_batch(5, "cpu", B=6, V=500)
    ref = bench.oracle_inputs(b, chunk=6)
    import oracle
    want = oracle.verify_batch(**ref[0])
    got = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in want.items()}
    got["p_draft"] = want["p_draft"].astype(np.float32)
    got["q_draft"] = want["q_draft"].astype(np.float32)
    assert bench.parity_summary(b, got, want)["mismatches"] == 0
    off = b.offsets
    stoch = [i for i in range(b.B) if not b.greedy[i]]
    greedy = [i for i in range(b.B) if b.greedy[i]]
    assert stoch and greedy
    s, g = stoch[0], greedy[0]
    bad = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in got.items()}
    slot = int(off[s]) + s + int(want["accepted_len"][s])
    bad["out_tokens"][slot] = (int(bad["out_tokens"][slot]) + 1) % b.V
    tight = dict(want, margin=want["margin"].copy())
    tight["margin"][s] = 5e-7
    r = bench.parity_summary(b, bad, tight)
    assert (r["mismatches"], r["near_ties"]) == (0, 1), r
    tight["margin"][s] = 2e-6
    r = bench.parity_summary(b, bad, tight)
    assert (r["mismatches"], r["near_ties"]) == (1, 0), r
    badg = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in got.items()}
    badg["accepted_len"][g] = int(badg["accepted_len"][g]) + 1
    r = bench.parity_summary(b, badg, want)
    assert (r["mismatches"], r["near_ties"]) == (1, 0), r
