"""Comparison of the HIP path with the fp64 oracle on the same batch.

Rule: per request, equal (accepted length, committed tokens) passes.  A
stochastic request may differ only when the oracle's smallest decision margin
is below 1e-6 relative (the ratio tests up to the cut, relative to the larger
side; the final inverse-CDF draw, relative to the total of its weights);
such near-ties are counted, returned and reported at the end of the session.
Greedy requests must always match exactly.  p(y), q(y) and the residual mass
must agree within 1e-5 absolute (fp32 outputs against fp64).
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synth

NEAR_TIE = 1e-6
PROB_TOL = 1e-5
# (label, request, oracle margin) of every near-tie met in this process
NEAR_TIES = []


def run_hip(batch: synth.Batch, **kw) -> dict:
    import draft_token_verification_row_amd as sv
    res = sv.verify_batch(batch, **kw)
    torch.cuda.synchronize()
    return {k: (None if v is None else v.cpu().numpy()) for k, v in res.items()}


def run_oracle(batch: synth.Batch, chunk: int = 0) -> dict:
    """The oracle on every request of the batch.  chunk > 0 runs it on
    consecutive groups of that many requests (host copies of one group at a
    time) and concatenates the results, which stay in the packed layout because
    requests are independent and the groups keep their order."""
    if chunk <= 0 or batch.B <= chunk:
        return oracle.verify_batch(**synth.as_numpy(batch))
    parts = []
    for s0 in range(0, batch.B, chunk):
        sub = synth.select_requests(batch, list(range(s0, min(s0 + chunk, batch.B))), device="cpu")
        parts.append(oracle.verify_batch(**synth.as_numpy(sub)))
    return {k: np.concatenate([p[k] for p in parts]) for k in parts[0]}


def compare(batch: synth.Batch, got: dict, ref: dict, label: str = "") -> int:
    B = batch.B
    nd = batch.num_draft.astype(np.int64)
    off = np.concatenate([[0], np.cumsum(nd)])
    near = 0
    for b in range(B):
        k = int(nd[b])
        sl = slice(int(off[b]) + b, int(off[b]) + b + k + 1)
        same = (int(got["accepted_len"][b]) == int(ref["accepted_len"][b])
                and np.array_equal(got["out_tokens"][sl].astype(np.int64), ref["out_tokens"][sl]))
        if same:
            continue
        msg = (f"{label} request {b} (k={k}, greedy={bool(batch.greedy[b])}): "
               f"gpu a={got['accepted_len'][b]} tokens={got['out_tokens'][sl].tolist()} | "
               f"oracle a={ref['accepted_len'][b]} tokens={ref['out_tokens'][sl].tolist()} "
               f"margin={ref['margin'][b]:.3e}")
        if batch.greedy[b] or not (ref["margin"][b] < NEAR_TIE):
            raise AssertionError(msg)
        near += 1
        NEAR_TIES.append((label, b, float(ref["margin"][b])))
        print(f"near-tie: {msg}", flush=True)
    if batch.temperature is not None and got.get("p_draft") is not None:
        stoch_rows = np.repeat(batch.greedy == 0, nd)
        for name in ("p_draft", "q_draft"):
            g, r = got[name].astype(np.float64), ref[name]
            bad = np.flatnonzero(np.abs(g - r) > PROB_TOL)
            assert bad.size == 0, f"{label} {name} rows {bad[:8]}: gpu {g[bad[:8]]} oracle {r[bad[:8]]}"
            assert np.all(g[~stoch_rows] == -1.0)
        rm_g, rm_r = got["resid_mass"].astype(np.float64), ref["resid_mass"]
        agree = got["accepted_len"] == ref["accepted_len"]
        bad = np.flatnonzero(agree & (np.abs(rm_g - rm_r) > PROB_TOL))
        assert bad.size == 0, f"{label} resid_mass {bad[:8]}: gpu {rm_g[bad[:8]]} oracle {rm_r[bad[:8]]}"
    return near
