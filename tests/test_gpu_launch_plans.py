"""The single-launch plan (one workgroup per request) and the multi-kernel plan
return the same bits, and both match the oracle (needs the GPU)."""
import numpy as np
import pytest
import torch

import synth
from tests.parity import compare, run_hip, run_oracle
from tests.test_gpu_parity import SMALL

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _with_plan(plan, batch, **kw):
    import draft_token_verification_row_amd as sv
    sv.spec_verify_set_launch_plan(plan)
    try:
        return run_hip(batch, **kw)
    finally:
        sv.spec_verify_set_launch_plan(0)


@pytest.mark.parametrize("label,cfg,kw", SMALL, ids=[s[0] for s in SMALL])
def test_plans_bit_identical(label, cfg, kw):
    batch = synth.make_batch(cfg, DEV, **kw)
    multi = _with_plan(1, batch)
    single = _with_plan(2, batch)
    for k in multi:
        if multi[k] is not None:
            assert np.array_equal(multi[k], single[k], equal_nan=True), (label, k)
    compare(batch, single, run_oracle(batch), label + " single-launch")


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_plans_at_full_size(cfg):
    """Forced single launch on a whole workload (large V, many units per
    workgroup) against the multi-kernel plan."""
    batch = synth.make_batch(cfg, DEV)
    multi = _with_plan(1, batch)
    single = _with_plan(2, batch)
    for k in multi:
        if multi[k] is not None:
            assert np.array_equal(multi[k], single[k], equal_nan=True), (cfg, k)


def test_single_launch_input_errors():
    import draft_token_verification_row_amd as sv
    batch = synth.make_batch(5, DEV, B=10, V=5000)
    nd = torch.as_tensor(batch.num_draft, dtype=torch.int32, device=DEV)
    gm = torch.as_tensor(batch.greedy, dtype=torch.uint8, device=DEV)
    sv.spec_verify_set_launch_plan(2)
    try:
        bad = nd.clone()
        bad[0] += 1
        r = sv.spec_verify_sample(batch.target, batch.draft, batch.tokens, bad, batch.temperature,
                                  batch.u_accept, batch.u_final, greedy_mask=gm)
        torch.cuda.synchronize()
        assert torch.all(r["accepted_len"] == -1) and torch.all(r["out_tokens"] == -1)
        assert torch.all(r["p_draft"] == -1) and torch.all(r["resid_mass"] == -1)
        toks = batch.tokens.clone()
        b0 = int(np.flatnonzero((batch.greedy == 0) & (batch.num_draft > 0))[0])
        toks[int(batch.offsets[b0])] = 5000
        r = sv.spec_verify_sample(batch.target, batch.draft, toks, nd, batch.temperature,
                                  batch.u_accept, batch.u_final, greedy_mask=gm)
        torch.cuda.synchronize()
        assert int(r["accepted_len"][b0]) == -1
    finally:
        sv.spec_verify_set_launch_plan(0)
