"""Planted mistakes in the oracle (CPU only) must each fail at least one pin.

This shows the pins constrain every step: the ratio test, the residual, the
inverse CDF, the temperature, the tie rule, row/operand indexing and the cut,
and the decision margins that classify GPU/oracle disagreements as near-ties.
"""
import numpy as np
import pytest

import oracle.verify as vm
from tests import oracle_pins as pins

_orig_request = vm.verify_request
_orig_cdf = vm.inverse_cdf
_orig_softmax = vm.tempered_softmax


def _cdf_left(weights, w):
    c = np.cumsum(weights)
    total = float(c[-1])
    hits = np.flatnonzero(c >= w * total)
    t = int(hits[0]) if hits.size else int(np.flatnonzero(weights > 0)[-1])
    return t, total, 1.0


def _cdf_descending(weights, w):
    t, total, m = _orig_cdf(np.asarray(weights)[::-1], w)
    return len(weights) - 1 - t, total, m


def _cdf_unscaled(weights, w):
    c = np.cumsum(weights)
    hits = np.flatnonzero(c > w)
    t = int(hits[0]) if hits.size else int(np.flatnonzero(weights > 0)[-1])
    return t, float(c[-1]), 1.0


def _bonus_from_previous_row(target_rows, draft_rows, tokens, greedy, T, u, w):
    t = np.array(target_rows, copy=True)
    if len(tokens) >= 1:
        t[len(tokens)] = t[len(tokens) - 1]
    return _orig_request(t, draft_rows, tokens, greedy, T, u, w)


def _q_from_target(target_rows, draft_rows, tokens, greedy, T, u, w):
    d = None if draft_rows is None else np.array(target_rows[:len(tokens)], copy=True)
    return _orig_request(target_rows, d, tokens, greedy, T, u, w)


def _uniforms_shifted(target_rows, draft_rows, tokens, greedy, T, u, w):
    return _orig_request(target_rows, draft_rows, tokens, greedy, T, np.roll(np.asarray(u), 1), w)


def _greedy_next_row(target_rows, draft_rows, tokens, greedy, T, u, w):
    t = np.array(target_rows, copy=True)
    if greedy and len(t) > 1:
        t = np.concatenate([t[1:], t[-1:]])
    return _orig_request(t, draft_rows, tokens, greedy, T, u, w)


def _no_cut(target_rows, draft_rows, tokens, greedy, T, u, w):
    r = _orig_request(target_rows, draft_rows, tokens, greedy, T, u, w)
    k = len(tokens)
    if r["a"] < k:      # keep the later drafts anyway
        r = dict(r, committed=r["committed"] + [int(x) for x in tokens[r["a"] + 1:]])
    return r


def _cdf_margin(edge_shift_lo=0, edge_shift_hi=0, scale=False, zero=False):
    """inverse_cdf with a mistaken margin: wrong interval edge, absolute
    instead of relative to the total, or always 0."""
    def f(weights, w):
        t, total, m = _orig_cdf(weights, w)
        c = np.concatenate([[0.0], np.cumsum(np.asarray(weights, np.float64))])
        thr = float(w) * total
        lo = c[min(max(t + edge_shift_lo, 0), len(c) - 1)]
        hi = c[min(max(t + 1 + edge_shift_hi, 0), len(c) - 1)]
        m = min(abs(lo - thr), abs(hi - thr)) / (1.0 if scale else total) if total > 0 else 0.0
        return t, total, 0.0 if zero else m
    return f


def _request_margin(mode):
    """verify_request whose margin leaves out the draw ("tests") or also takes
    the ratio tests after the cut ("all")."""
    def f(target_rows, draft_rows, tokens, greedy, T, u, w):
        r = _orig_request(target_rows, draft_rows, tokens, greedy, T, u, w)
        if greedy or len(tokens) == 0:
            return r
        k, a = len(tokens), r["a"]
        ms = [vm.accept_margin(u[i], r["p_y"][i], r["q_y"][i]) for i in range(k)]
        if mode == "tests":
            m = min(ms[:min(a + 1, k)])
        else:
            m = min([r["margin"]] + ms)
        return dict(r, margin=m)
    return f


MUTANTS = {
    "accept_margin_zero": ("accept_margin", lambda u, p, q: 0.0),
    "accept_margin_absolute": ("accept_margin", lambda u, p, q: abs(float(u) * q - p)),
    "draw_margin_zero": ("inverse_cdf", _cdf_margin(zero=True)),
    "draw_margin_absolute": ("inverse_cdf", _cdf_margin(scale=True)),
    "draw_margin_next_upper_edge": ("inverse_cdf", _cdf_margin(edge_shift_hi=1)),
    "draw_margin_previous_lower_edge": ("inverse_cdf", _cdf_margin(edge_shift_lo=-1)),
    "request_margin_without_draw": ("verify_request", _request_margin("tests")),
    "request_margin_after_cut": ("verify_request", _request_margin("all")),
    "accept_le": ("keeps_draft", lambda u, p, q: float(u) * q <= p),
    "accept_swapped": ("keeps_draft", lambda u, p, q: float(u) * p < q),
    "accept_inverted": ("keeps_draft", lambda u, p, q: float(u) * q > p),
    "accept_always": ("keeps_draft", lambda u, p, q: True),
    "residual_transposed": ("positive_residual", lambda p, q: np.maximum(q - p, 0.0)),
    "residual_unclamped": ("positive_residual", lambda p, q: np.abs(p - q)),
    "residual_is_target": ("positive_residual", lambda p, q: p),
    "cdf_left_side": ("inverse_cdf", _cdf_left),
    "cdf_descending": ("inverse_cdf", _cdf_descending),
    "cdf_unscaled_threshold": ("inverse_cdf", _cdf_unscaled),
    "temperature_not_widened": ("widen_temperature", lambda T: float(T)),
    "softmax_ignores_T": ("tempered_softmax", lambda z, T: _orig_softmax(z, 1.0)),
    "softmax_times_T": ("tempered_softmax", lambda z, T: _orig_softmax(np.asarray(z) * T * T, T)),
    "argmax_highest_id": ("lowest_argmax",
                          lambda z: int(np.flatnonzero(np.asarray(z) == np.max(z))[-1])),
    "bonus_from_previous_row": ("verify_request", _bonus_from_previous_row),
    "q_from_target_rows": ("verify_request", _q_from_target),
    "uniforms_shifted": ("verify_request", _uniforms_shifted),
    "greedy_next_row": ("verify_request", _greedy_next_row),
    "no_cut_at_reject": ("verify_request", _no_cut),
}


def _fast_mc(v):
    pins.pin_monte_carlo(v, trials=3000, cases=((3, 3), (8, 1)), seed=2)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(vm, attr, fn)
    caught = None
    for pin in pins.ALL_PINS + [_fast_mc]:
        try:
            pin(vm)
        except Exception as e:  # an assertion, or a crash the mistake provokes
            caught = (pin.__name__, type(e).__name__)
            break
    assert caught is not None, f"mutant {name} passed every pin"
