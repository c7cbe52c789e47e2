"""Acceptance statistics on the GPU against the oracle (needs the GPU)."""
import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle.accept_stats as am
import synth
from tests.parity import run_hip

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _gpu_stats(acc, nd, max_pos):
    import draft_token_verification_row_amd as sv
    out = sv.spec_verify_accept_stats(acc, nd, max_pos)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _same(got, st, max_pos):
    assert got[0] == st["rounds"]
    assert got[1] == st["mean_accepted"] and got[2] == st["mal"] and got[3] == st["ar"]
    assert np.array_equal(got[4:4 + max_pos], st["per_position"])


@pytest.mark.parametrize("cfg,kw,max_pos", [(5, dict(B=300, V=4000), 8), (4, dict(B=16, V=3000), 15),
                                             (2, dict(B=64, V=2000), 3), (5, dict(B=300, V=4000), 3)])
def test_stats_of_a_verification_call(cfg, kw, max_pos):
    batch = synth.make_batch(cfg, DEV, **kw)
    got = run_hip(batch)
    acc = torch.as_tensor(got["accepted_len"], device=DEV)
    nd = torch.as_tensor(batch.num_draft, dtype=torch.int32, device=DEV)
    _same(_gpu_stats(acc, nd, max_pos), am.acceptance_stats(got["accepted_len"], batch.num_draft, max_pos),
          max_pos)


def test_hand_ragged_case_on_gpu():
    acc = torch.tensor([2, 1, 0, 0, -1], dtype=torch.int32, device=DEV)
    nd = torch.tensor([3, 1, 0, 2, 5], dtype=torch.int32, device=DEV)
    got = _gpu_stats(acc, nd, 4)
    assert got[0] == 4 and got[1] == 0.75 and got[2] == 1.75 and got[3] == 0.5
    assert np.allclose(got[4:], [2 / 3, 0.5, 0.0, -1.0], rtol=0, atol=1e-15)


def test_survival_matches_closed_form():
    """Many requests over the same small rows: per-position acceptance estimates
    P(A >= j) = prod_{i<j} beta_i and MAL estimates DSpark's progress formula."""
    import oracle
    rng = np.random.default_rng(77)
    V, k, N, T = 16, 5, 100000, 1.0
    z = rng.normal(0, 1.5, size=(k + 1, V)).astype(np.float32)
    d = (z[:k] + rng.normal(0, 0.7, size=(k, V))).astype(np.float32)
    P = [scipy.special.softmax(z[i].astype(np.float64) / T) for i in range(k + 1)]
    Q = [scipy.special.softmax(d[i].astype(np.float64) / T) for i in range(k)]
    beta = [float(np.minimum(P[i], Q[i]).sum()) for i in range(k)]
    ys = np.stack([np.minimum(np.searchsorted(np.cumsum(Q[i]), rng.random(N), side="right"), V - 1)
                   for i in range(k)], axis=1)
    batch = synth.Batch(
        name="mc", B=N, K=N * k, V=V, dtype="f32", num_draft=np.full(N, k, np.int32),
        greedy=np.zeros(N, np.uint8), temperature=T,
        target=torch.as_tensor(np.tile(z, (N, 1)), device=DEV),
        draft=torch.as_tensor(np.tile(d, (N, 1)), device=DEV),
        tokens=torch.as_tensor(ys.reshape(-1).astype(np.int32), device=DEV),
        u_accept=torch.as_tensor(synth.uniforms_f32(rng, N * k), device=DEV),
        u_final=torch.as_tensor(synth.uniforms_f32(rng, N), device=DEV))
    got = run_hip(batch, want_probs=False)
    st = _gpu_stats(torch.as_tensor(got["accepted_len"], device=DEV),
                    torch.as_tensor(batch.num_draft, device=DEV), k)
    for j in range(1, k + 1):
        surv = float(np.prod(beta[:j]))
        sd = math.sqrt(surv * (1 - surv) / N)
        assert abs(st[3 + j] - surv) <= 5 * sd + 1e-9, (j, st[3 + j], surv)
    prog = oracle.expected_progress(beta, k)
    a = got["accepted_len"].astype(np.float64)
    assert abs(st[2] - prog) <= 5 * math.sqrt(a.var() / N)
