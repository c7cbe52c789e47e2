"""Draws from residuals far smaller than fp32 can resolve (needs the GPU).

The draft row equals the target row except at one id j, raised by delta, and
the draft token is j: the ratio test rejects it (u just below 1), and the
residual [p - q]_+ has total q_j - p_j, which is tiny when j lies deep in the
target's tail.  Its weights are p_v - q_v for every other id: differences of
nearly equal probabilities that fp32 evaluations of p and q cannot resolve, so
the library must redo such draws in fp64.  The GPU must match the oracle under
the relative near-tie rule, through both launch plans and early exit.  Also
moderate totals (1e-4 .. 1e-2), bonus draws near an interval edge, and one
request at V = 262144.
"""
import sys

import numpy as np
import pytest
import torch

import synth
from tests.parity import compare, run_hip, run_oracle
from tests.test_gpu_early_exit import _oracle_as_tested

pytestmark = pytest.mark.gpu
DEV = "cuda"
U_REJECT = float(np.float32(1.0 - 2.0 ** -24))      # largest fp32 below 1


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _tiny_residual_batch(V, dtype, deltas, seed, ws=None, T=1.0, k_extra=1, where="tail"):
    """One request per delta: position 0 carries the bump (rejected) at the
    target's lowest logit (where="tail": residual total ~ p_j * delta, far
    below fp32 resolution) or at its highest (where="peak": moderate totals);
    positions after it are ordinary rows (never reached)."""
    rng = np.random.default_rng(seed)
    B = len(deltas)
    ks = [1 + k_extra] * B
    K = sum(ks)
    off = np.concatenate([[0], np.cumsum(ks)])
    tgt = rng.normal(0, 2.0, size=(K + B, V)).astype(np.float32)
    tgt = torch.as_tensor(tgt).to(synth.TORCH_DTYPE[dtype]).to(torch.float32).numpy()
    drf = np.zeros((K, V), np.float32)
    toks = np.zeros(K, np.int64)
    for b, delta in enumerate(deltas):
        for i in range(ks[b]):
            t = tgt[off[b] + b + i]
            if i == 0:
                j = int(np.argmin(t)) if where == "tail" else int(np.argmax(t))
                d = t.copy()
                d[j] = t[j] + delta
                d = torch.as_tensor(d).to(synth.TORCH_DTYPE[dtype]).to(torch.float32).numpy()
                assert d[j] != t[j]
                y = j
            else:
                d = t + rng.normal(0, 1.0, size=V).astype(np.float32)
                y = int(rng.integers(V))
            drf[off[b] + i] = d
            toks[off[b] + i] = y
    u = np.full(K, 0.5, np.float32)
    u[off[:-1]] = U_REJECT
    uf = np.asarray(ws if ws is not None else rng.random(B), np.float32)
    return synth.from_arrays(tgt, drf, toks, ks, greedy=[0] * B, temperature=T, u_accept=u,
                             u_final=uf, dtype=dtype, name="tiny_residual", device=DEV)


def _all_paths(batch, label):
    import draft_token_verification_row_amd as sv
    ref = run_oracle(batch)
    outs = {}
    for name, plan in (("multi", 1), ("single", 2)):
        sv.spec_verify_set_launch_plan(plan)
        try:
            outs[name] = run_hip(batch)
        finally:
            sv.spec_verify_set_launch_plan(0)
    outs["early_exit"] = run_hip(batch, max_k=int(batch.num_draft.max()))
    for name, got in outs.items():
        want = _oracle_as_tested(batch, got, ref) if name == "early_exit" else ref
        near = compare(batch, got, want, f"{label} {name}")
        _log(f"[certified] {label} {name}: near_ties={near}")
    for k in ("accepted_len", "out_tokens", "resid_mass"):
        assert np.array_equal(outs["multi"][k], outs["single"][k]), k
        assert np.array_equal(outs["multi"][k], outs["early_exit"][k]), k
    return ref, outs["multi"]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_residual_totals_below_fp32_resolution(dtype):
    deltas = [0.5, 1.0, 2.0, 4.0, 8.0] * 2
    ws = np.linspace(0.03, 0.97, len(deltas))
    batch = _tiny_residual_batch(5003, dtype, deltas, seed=11, ws=ws)
    ref, got = _all_paths(batch, f"tiny {dtype}")
    Z = ref["resid_mass"]
    _log(f"[certified] residual totals {np.array2string(Z, precision=2)}")
    assert np.all(ref["accepted_len"] == 0) and np.all(Z < 1e-3) and np.all(Z > 0)
    # totals far below fp32 resolution come from the fp64 draw, which reports
    # its own total: relative agreement, not only the 1e-5 absolute of fp32
    tiny = Z < 1e-6
    rel = np.abs(got["resid_mass"].astype(np.float64) - Z)[tiny] / Z[tiny]
    assert tiny.sum() >= 4 and np.all(rel < 1e-5), rel


def test_moderate_residual_totals():
    """Bumps at the target's peak: totals of about 1e-4 .. 1e-2, where fp32
    weights are accurate to a few 1e-7 of the mass and most crossings are
    certified."""
    rng = np.random.default_rng(3)
    deltas = [0.01, 0.03, 0.1, 0.3, 0.6] * 4
    ws = rng.random(len(deltas))
    batch = _tiny_residual_batch(20011, "f32", deltas, seed=12, ws=ws, where="peak")
    ref, _ = _all_paths(batch, "moderate")
    _log(f"[certified] moderate totals {np.array2string(ref['resid_mass'], precision=2)}")


def test_draws_near_an_interval_edge():
    """Uniforms placed within 1e-9 .. 1e-5 of a cumulative edge of the bonus
    distribution (k = 0): the fp32 draw is kept for draws from p, so this
    checks its accuracy where it matters most: every draw whose exact margin
    is 1e-6 of the total or more must match the oracle."""
    import scipy.special
    rng = np.random.default_rng(21)
    V, B = 4099, 24
    z = rng.normal(0, 2.0, size=(B, V)).astype(np.float32)
    ws = []
    for b in range(B):
        p = scipy.special.softmax(z[b].astype(np.float64))
        c = np.cumsum(p)
        t = int(rng.integers(10, V - 10))
        off = [1e-5, 1e-6, 1e-7, 3e-8, 1e-9, -1e-9, -1e-7, -1e-5][b % 8]
        ws.append(float(np.float32(c[t] / c[-1] + off)))
    batch = synth.from_arrays(z, np.zeros((0, V), np.float32), np.zeros(0, np.int64), [0] * B,
                              greedy=[0] * B, temperature=1.0, u_accept=np.zeros(0, np.float32),
                              u_final=ws, dtype="f32", name="edge", device=DEV)
    _all_paths(batch, "edge")


def test_tiny_residual_at_full_vocabulary():
    """One request with V = 262144 bf16 (the fp64 draw sweeps the pair on one CU)."""
    batch = _tiny_residual_batch(262144, "bf16", [2.0, 1.0], seed=5, ws=[0.37, 0.81])
    _all_paths(batch, "V=262144")
