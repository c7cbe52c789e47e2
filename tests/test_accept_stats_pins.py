"""Acceptance statistics (oracle) against the pages' Appendix tables (CPU only)."""
import numpy as np
import pytest

import oracle.accept_stats as am
from tests import oracle_pins as pins


def test_appendix_identities():
    pins.pin_acceptance_appendix(am)


def test_ragged_hand_case():
    pins.pin_acceptance_ragged(am)


def _mal_without_final(a, k, m):
    st = am_orig(a, k, m)
    st["mal"] -= 1.0
    return st


def _ar_over_max(a, k, m):
    st = am_orig(a, k, m)
    a, k = np.asarray(a), np.asarray(k)
    ok = a >= 0
    st["ar"] = a[ok].sum() / (ok.sum() * max(int(k.max()), 1))
    return st


def _per_position_over_all(a, k, m):
    st = am_orig(a, k, m)
    a = np.asarray(a)
    a = a[a >= 0]
    st["per_position"] = np.array([(a >= j).sum() / a.size for j in range(1, m + 1)])
    return st


def _per_position_strict(a, k, m):
    st = am_orig(a, k, m)
    a, k = np.asarray(a), np.asarray(k)
    ok = a >= 0
    a, k = a[ok], k[ok]
    st["per_position"] = np.array([((a > j).sum() / max((k >= j).sum(), 1)) for j in range(1, m + 1)])
    return st


am_orig = am.acceptance_stats
MUTANTS = {"mal_without_final_token": _mal_without_final, "ar_over_max_k": _ar_over_max,
           "per_position_over_all_rounds": _per_position_over_all,
           "per_position_strict": _per_position_strict}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    monkeypatch.setattr(am, "acceptance_stats", MUTANTS[name])
    caught = False
    for pin in pins.ACCEPT_PINS:
        try:
            pin(am)
        except AssertionError:
            caught = True
            break
    assert caught, name
