"""Large-size cases against the oracle (needs the GPU).

* a vocabulary of 2^27 ids (8192 row units of 32 KiB, 32768 residual units per
  row pair): every unit count, combine loop and unit search at its widest;
* 65536 requests in one call (offset scan over 64 chunks, 16384 decide
  blocks, 65536 draw blocks);
each through the multi-kernel plan, the single launch and early exit.
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


def _plans(batch):
    import draft_token_verification_row_amd as sv
    out = {}
    for plan in (1, 2):
        sv.spec_verify_set_launch_plan(plan)
        try:
            out[plan] = run_hip(batch)
        finally:
            sv.spec_verify_set_launch_plan(0)
    out["ee"] = run_hip(batch, max_k=int(batch.num_draft.max(initial=0)))
    return out


@pytest.mark.timeout(400)
def test_vocabulary_2_pow_27():
    _log("[limits] V = 2^27 generating")
    batch = synth.make_batch(5, DEV, B=3, V=1 << 27, k=2, seed=77)
    torch.cuda.synchronize()
    _log(f"[limits] V = 2^27: B={batch.B} K={batch.K} greedy={batch.greedy.tolist()} running")
    got = _plans(batch)
    ref = run_oracle(batch)
    for name in (1, 2):
        near = compare(batch, got[name], ref, f"V=2^27 plan {name}")
    for k in ("accepted_len", "out_tokens", "resid_mass"):
        assert np.array_equal(got[1][k], got[2][k]), k
        assert np.array_equal(got[1][k], got["ee"][k]), k
    _log(f"[limits] V = 2^27: accepted {got[1]['accepted_len'].tolist()}")


@pytest.mark.timeout(400)
def test_65536_requests():
    _log("[limits] B = 65536 generating")
    batch = synth.make_batch(5, DEV, B=65536, V=64, seed=78)
    torch.cuda.synchronize()
    _log(f"[limits] B = 65536: K={batch.K} running")
    got = _plans(batch)
    ref = run_oracle(batch)
    near = compare(batch, got[1], ref, "B=65536")
    n_stoch = int((batch.greedy == 0).sum())
    for k in ("accepted_len", "out_tokens", "resid_mass", "p_draft", "q_draft"):
        assert np.array_equal(got[1][k], got[2][k]), k
    for k in ("accepted_len", "out_tokens", "resid_mass"):
        assert np.array_equal(got[1][k], got["ee"][k]), k
    _log(f"[limits] B = 65536: near ties {near}, mean accepted {got[1]['accepted_len'].mean():.3f}")
