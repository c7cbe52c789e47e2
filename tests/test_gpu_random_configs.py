"""Broad parity sweep over seeded random configurations (synth.make_random_batch:
dtype, vocabulary, ragged k, greedy share, temperature, logit scale, strided
rows, masked columns) against the fp64 oracle, through both launch plans of the
all-rows entry points (bit for bit equal to each other) and through early exit
(bit for bit equal to the all-rows path at the tested positions).  Needs the GPU."""
import os
import sys

import numpy as np
import pytest
import torch

import synth
from tests.parity import compare, run_hip, run_oracle

pytestmark = pytest.mark.gpu
DEV = "cuda"
# SPEC_VERIFY_RANDOM_SEEDS="lo:hi" sweeps other seeds (default the first 150)
_lo, _hi = (int(x) for x in os.environ.get("SPEC_VERIFY_RANDOM_SEEDS", "0:150").split(":"))
SEEDS = list(range(_lo, _hi))


def _plan(sv, plan, batch):
    sv.spec_verify_set_launch_plan(plan)
    try:
        return run_hip(batch)
    finally:
        sv.spec_verify_set_launch_plan(0)


@pytest.mark.parametrize("seed", SEEDS)
def test_random_configuration(seed):
    import draft_token_verification_row_amd as sv
    batch = synth.make_random_batch(seed, DEV)
    torch.cuda.synchronize()
    print(f"[random] seed={seed} {batch.dtype} B={batch.B} K={batch.K} V={batch.V} "
          f"T={batch.temperature:.4g} greedy={int(batch.greedy.sum())} "
          f"ld={batch.target.stride(0)}", flush=True)
    sys.stdout.flush()
    ref = run_oracle(batch)
    multi = _plan(sv, 1, batch)
    single = _plan(sv, 2, batch)
    n_stoch = int((batch.greedy == 0).sum())
    for name, got in (("multi", multi), ("single", single)):
        near = compare(batch, got, ref, f"seed {seed} {name}")
    for k in multi:
        if multi[k] is not None:
            assert np.array_equal(multi[k], single[k]), (seed, k)
    max_k = int(batch.num_draft.max(initial=0)) + seed % 3
    ee = run_hip(batch, max_k=max_k)
    for k in ("accepted_len", "out_tokens", "resid_mass"):
        assert np.array_equal(ee[k], multi[k]), (seed, k)
    nd = batch.num_draft.astype(np.int64)
    off = np.concatenate([[0], np.cumsum(nd)])
    for b in range(batch.B):
        if batch.greedy[b] or ee["accepted_len"][b] < 0:
            continue
        n = min(int(ee["accepted_len"][b]) + 1, int(nd[b]))
        s = slice(int(off[b]), int(off[b]) + n)
        assert np.array_equal(ee["p_draft"][s], multi["p_draft"][s]), (seed, b)
        assert np.array_equal(ee["q_draft"][s], multi["q_draft"][s]), (seed, b)
