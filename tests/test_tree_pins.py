"""Tree-walk oracle against its pins, and planted mistakes that the pins catch (CPU)."""
import numpy as np
import pytest

import oracle.tree as ot
import oracle.verify as ov
from tests import tree_pins as tp


@pytest.mark.parametrize("pin", tp.TREE_PINS, ids=[p.__name__ for p in tp.TREE_PINS])
def test_tree_pin(pin):
    pin()


_orig_walk = ot.tree_walk_greedy


def _child_row(target_rows, parent, tokens):
    """compares a child's token with the choice on the child's own row"""
    kids = ot.children_of(parent)
    path, committed, cur = [0], [], 0
    while True:
        follow = None
        for c in kids[cur]:
            if int(tokens[c]) == ov.lowest_argmax(target_rows[c]):
                follow = c
                break
        if follow is None:
            committed.append(ov.lowest_argmax(target_rows[cur]))
            break
        committed.append(int(tokens[follow])); path.append(follow); cur = follow
    return dict(a=len(path) - 1, path=path, committed=committed)


def _highest_duplicate(target_rows, parent, tokens):
    kids = ot.children_of(parent)
    rev = list(parent)
    path, committed, cur = [0], [], 0
    while True:
        ch = ov.lowest_argmax(target_rows[cur])
        m = [c for c in kids[cur] if int(tokens[c]) == ch]
        if not m:
            committed.append(ch)
            break
        committed.append(ch); path.append(m[-1]); cur = m[-1]
    return dict(a=len(path) - 1, path=path, committed=committed)


def _bonus_from_root(target_rows, parent, tokens):
    r = _orig_walk(target_rows, parent, tokens)
    r["committed"][-1] = ov.lowest_argmax(target_rows[0])
    return r


def _counts_root(target_rows, parent, tokens):
    r = _orig_walk(target_rows, parent, tokens)
    r["a"] = len(r["path"])
    return r


def _stops_after_one(target_rows, parent, tokens):
    r = _orig_walk(target_rows, parent, tokens)
    if r["a"] > 1:
        cur = r["path"][1]
        r = dict(a=1, path=r["path"][:2],
                 committed=r["committed"][:1] + [ov.lowest_argmax(target_rows[cur])])
    return r


def _highest_tie(target_rows, parent, tokens):
    orig = ov.lowest_argmax
    try:
        ot.lowest_argmax = lambda z: int(np.flatnonzero(np.asarray(z) == np.max(z))[-1])
        return _orig_walk(target_rows, parent, tokens)
    finally:
        ot.lowest_argmax = orig


def _no_parent_check(target_rows, parent, tokens):
    orig = ot.check_parents
    try:
        ot.check_parents = lambda p: None
        return _orig_walk(target_rows, parent, tokens)
    finally:
        ot.check_parents = orig


MUTANTS = [_child_row, _highest_duplicate, _bonus_from_root, _counts_root, _stops_after_one,
           _highest_tie, _no_parent_check]


@pytest.mark.parametrize("mutant", MUTANTS, ids=[m.__name__ for m in MUTANTS])
def test_tree_mutant_is_caught(mutant, monkeypatch):
    monkeypatch.setattr(ot, "tree_walk_greedy", mutant)
    failed = []
    for pin in tp.TREE_PINS:
        try:
            pin()
        except Exception:           # noqa: BLE001 - any failure counts
            failed.append(pin.__name__)
    assert failed, f"{mutant.__name__} passed every pin"
