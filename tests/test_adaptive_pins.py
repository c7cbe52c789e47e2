"""Adaptive-length oracle against its pins, and planted mistakes the pins catch (CPU)."""
import numpy as np
import pytest

import oracle.adaptive as oa
from tests import adaptive_pins as ap


@pytest.mark.parametrize("pin", ap.ADAPTIVE_PINS, ids=[p.__name__ for p in ap.ADAPTIVE_PINS])
def test_adaptive_pin(pin):
    pin()


_orig_prog = oa.progress_table
_orig_choose = oa.choose_length
_orig_batch = oa.adaptive_batch


def _ties_largest(conf, cost):
    prog = _orig_prog(conf)
    r = [prog[k] / float(cost[k]) for k in range(len(prog))]
    k = max(i for i in range(len(r)) if r[i] == max(r))
    return k, float(prog[k])


def _no_leading_one(conf):
    return _orig_prog(conf) - 1.0


def _shifted_conf(conf):
    c = list(conf[1:]) + [1.0]
    return _orig_prog(np.asarray(c, np.float32))


def _cost_shift(conf, cost):
    c = list(cost[1:]) + [cost[-1]]
    return _orig_choose(conf, c)


def _suffix_window(conf, cost, tokens):
    r = _orig_batch(conf, cost, tokens)
    N = np.asarray(conf).shape[1]
    src = []
    for b, k in enumerate(r["num_draft"]):
        src.extend(b * N + np.arange(N - k, N))
    r["src_index"] = np.array(src, np.int64)
    r["tokens"] = np.asarray(tokens).reshape(-1)[r["src_index"]] if src else r["tokens"]
    return r


def _inclusive_offsets(conf, cost, tokens):
    r = _orig_batch(conf, cost, tokens)
    r["offsets"] = np.concatenate([np.cumsum(r["num_draft"]), [r["offsets"][-1]]])
    return r


def _squared_survival(conf):
    return _orig_prog(np.asarray(conf, np.float32) ** 2)


MUTANTS = [("choose_length", _ties_largest), ("progress_table", _no_leading_one),
           ("progress_table", _shifted_conf), ("choose_length", _cost_shift),
           ("adaptive_batch", _suffix_window), ("adaptive_batch", _inclusive_offsets),
           ("progress_table", _squared_survival)]


@pytest.mark.parametrize("attr,mutant", MUTANTS, ids=[m[1].__name__ for m in MUTANTS])
def test_adaptive_mutant_is_caught(attr, mutant, monkeypatch):
    monkeypatch.setattr(oa, attr, mutant)
    failed = []
    for pin in ap.ADAPTIVE_PINS:
        try:
            pin()
        except Exception:           # noqa: BLE001 - any failure counts
            failed.append(pin.__name__)
    assert failed, f"{mutant.__name__} passed every pin"
