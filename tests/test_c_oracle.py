"""The fp64 C oracle (oracle/verify_ref.c) against the pins and against the
NumPy oracle (CPU only).

The C oracle is the same definition written a second time, in C.  The pins
that fix the NumPy oracle (worked examples of the pages, exact quadrature,
Monte Carlo, special cases, margins) must hold for it too.  On seeded
workloads the two must agree on every accepted length and committed token,
on p(y), q(y) and the residual totals within 1e-12, and on the deciding
margins within 1e-9: they differ only in the order of the softmax sum
(sequential here, pairwise in NumPy) and in the exp() implementation, a few
units in the last place.
"""
import math

import numpy as np
import pytest

import oracle.verify as vm
import oracle.verify_c as vc
import synth
from tests import oracle_pins as pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=[p.__name__ for p in pins.ALL_PINS])
def test_pins_hold_for_the_c_oracle(pin):
    pin(vc)


def test_monte_carlo_pin_for_the_c_oracle():
    pins.pin_monte_carlo(vc, trials=6000)


def _agree(batch_np: dict, label: str, threads: int = 2):
    ref = vm.verify_batch(**batch_np)
    got = vc.verify_batch(**batch_np, threads=threads)
    nd = np.asarray(batch_np["num_draft"], np.int64)
    off = np.concatenate([[0], np.cumsum(nd)])
    assert np.array_equal(got["accepted_len"], ref["accepted_len"]), label
    for b in range(nd.size):
        sl = slice(int(off[b]) + b, int(off[b]) + b + int(nd[b]) + 1)
        assert np.array_equal(got["out_tokens"][sl], ref["out_tokens"][sl]), (label, b)
    assert np.array_equal(got["out_tokens"], ref["out_tokens"]), label
    for key in ("p_draft", "q_draft"):
        neg = ref[key] < 0
        assert np.array_equal(got[key] < 0, neg), (label, key)
        assert np.all(np.abs(got[key][~neg] - ref[key][~neg]) <= 1e-12), (label, key)
    z_ref, z_got = ref["resid_mass"], got["resid_mass"]
    assert np.array_equal(z_got < 0, z_ref < 0), label
    assert np.all(np.abs(z_got - z_ref) <= 1e-12 * np.maximum(1.0, np.abs(z_ref))), label
    fin = np.isfinite(ref["margin"])
    assert np.array_equal(np.isfinite(got["margin"]), fin), label
    assert np.all(np.abs(got["margin"][fin] - ref["margin"][fin]) <= 1e-9), label
    return got, ref


WORKLOADS = [
    ("tiny_full", 1, {}),
    ("greedy_V32000", 2, dict(B=16, V=32000)),
    ("f32_V40003", 3, dict(B=6, V=40003)),
    ("block16_bf16", 4, dict(B=2, V=20011)),
    ("mixed_V70001", 5, dict(B=16, V=70001)),
    ("mixed_strided", 5, dict(B=8, V=9999, target_ld=10001)),
    ("k0_all", 5, dict(B=12, V=5000, k=0)),
    ("block16_tiny_vocab", 4, dict(B=40, V=64)),
    ("f32_vocab_1", 3, dict(B=4, V=1, k=2)),
    ("mixed_many_requests", 5, dict(B=600, V=300)),
]


@pytest.mark.parametrize("label,cfg,kw", WORKLOADS, ids=[w[0] for w in WORKLOADS])
def test_agrees_with_the_numpy_oracle(label, cfg, kw):
    batch = synth.make_batch(cfg, "cpu", **kw)
    _agree(synth.as_numpy(batch), label)


@pytest.mark.parametrize("seed", range(24))
def test_agrees_on_random_configurations(seed):
    batch = synth.make_random_batch(seed, "cpu", max_elems=1 << 20)
    _agree(synth.as_numpy(batch), f"random_{seed}")


def test_fp64_logits_agree():
    """fp64 logits (the pins' input type) go through the same code."""
    rng = np.random.default_rng(4)
    B, V = 9, 777
    ks = rng.integers(0, 5, size=B)
    K = int(ks.sum())
    tgt = rng.normal(0, 2.0, size=(K + B, V))
    dr = rng.normal(0, 2.0, size=(K, V))
    d = dict(target=tgt, draft=dr, tokens=rng.integers(0, V, size=K), num_draft=ks,
             greedy=rng.random(B) < 0.3, temperature=0.6, u_accept=rng.random(K),
             u_final=rng.random(B))
    _agree(d, "fp64")


def test_thread_count_changes_no_bit():
    d = synth.as_numpy(synth.make_batch(5, "cpu", B=40, V=3001))
    one = vc.verify_batch(**d, threads=1)
    for t in (3, 8):
        many = vc.verify_batch(**d, threads=t)
        for key in one:
            assert np.array_equal(one[key], many[key]), (t, key)


def test_early_exit_form_of_the_c_oracle():
    """Distributions formed only when a test is reached: the same decisions,
    tokens, totals and margins; p(y), q(y) at the tested positions, -1 after."""
    d = synth.as_numpy(synth.make_batch(5, "cpu", B=32, V=4099))
    full = vc.verify_batch(**d, threads=2)
    ee = vc.verify_batch(**d, threads=2, early_exit=True)
    for key in ("accepted_len", "out_tokens", "resid_mass", "margin"):
        assert np.array_equal(full[key], ee[key]), key
    nd = d["num_draft"]
    off = np.concatenate([[0], np.cumsum(nd)])
    for b in range(nd.size):
        if d["greedy"][b]:
            continue
        n = min(int(full["accepted_len"][b]) + 1, int(nd[b]))
        s0 = slice(int(off[b]), int(off[b]) + n)
        s1 = slice(int(off[b]) + n, int(off[b + 1]))
        assert np.array_equal(ee["p_draft"][s0], full["p_draft"][s0])
        assert np.all(ee["p_draft"][s1] == -1.0) and np.all(ee["q_draft"][s1] == -1.0)
    ref = vm.verify_batch(**d, early_exit=True)
    assert np.array_equal(ee["accepted_len"], ref["accepted_len"])
    assert np.array_equal(ee["p_draft"] < 0, ref["p_draft"] < 0)


def test_invalid_stochastic_token_is_refused():
    z = np.zeros((2, 5))
    with pytest.raises(ValueError):
        vc.verify_request(z, z[:1], np.array([7]), False, 1.0, np.array([0.5]), 0.5)
    # a greedy request's tokens are only compared with the argmax
    r = vc.verify_request(z, None, np.array([7]), True, None, np.array([0.5]), 0.5)
    assert r["a"] == 0 and r["committed"] == [0] and math.isinf(r["margin"])
