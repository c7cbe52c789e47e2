"""Pins of the tree-walk oracle to facts that do not come from the oracle itself.

* a hand-derived example of the walk rule of chzhyang, "Speculative Decoding:
  ...", section 5 DDTree (tests/golden/tree_walk_example.json);
* a chain (every node has one child) is linear greedy verification, so the
  walk must agree with the linear oracle's greedy rule ([CZ] section 1);
* brute force: the accepted nodes are exactly the nodes whose whole ancestry
  is consistent (each node's token equals the target's choice at its parent);
  that set is a path from the root when siblings carry distinct tokens, and
  the bonus is the choice at its deepest node;
* a parent index outside [0, node) makes the request invalid.
Every pin calls the oracle through its module, so a planted mistake there is
seen here.
"""
import json
import os

import numpy as np

import oracle.tree as ot
import oracle.verify as ov

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tree_walk_example.json")


def _rows_from_case(case, n, V):
    rows = np.zeros((n, V))
    rows[:, 0] = 1.0
    for k, v in case["rows"].items():
        rows[int(k)] = v
    return rows


def pin_golden_tree():
    g = json.load(open(GOLDEN))
    parent, tokens = g["tree"]["parent"], g["tree"]["tokens"]
    for case in g["cases"]:
        rows = _rows_from_case(case, len(parent), g["vocab_size"])
        r = ot.tree_walk_greedy(rows, parent, tokens)
        assert r["a"] == case["accepted_len"], (case["name"], r)
        assert r["path"] == case["path"], (case["name"], r)
        assert r["committed"] == case["committed"], (case["name"], r)
    # a lone root commits the target's choice and nothing else
    r = ot.tree_walk_greedy(np.array([[0.0, 0.0, 2.0]]), [-1], [7])
    assert r == dict(a=0, path=[0], committed=[2])


def pin_chain_is_linear_greedy():
    rng = np.random.default_rng(11)
    for _ in range(300):
        k = int(rng.integers(0, 7))
        V = int(rng.integers(2, 6))
        rows = rng.integers(0, 3, size=(k + 1, V)).astype(float)     # ties on purpose
        toks = rng.integers(0, V, size=k)
        parent = [-1] + list(range(k))
        tree = ot.tree_walk_greedy(rows, parent, [0] + list(toks))
        lin = ov.verify_request(rows, None, toks, True, None, np.zeros(k), 0.0)
        assert tree["a"] == lin["a"], (rows, toks, tree, lin)
        assert tree["committed"] == lin["committed"]
        assert tree["path"] == list(range(tree["a"] + 1))


def _random_tree(rng, n, V):
    parent = [-1] + [int(rng.integers(0, i)) for i in range(1, n)]
    tokens = [int(rng.integers(0, V))]
    for i in range(1, n):
        sib = {tokens[j] for j in range(1, i) if parent[j] == parent[i]}
        free = [t for t in range(V) if t not in sib]
        tokens.append(int(rng.choice(free)) if free else -1)
    return parent, tokens


def _brute_force(rows, parent, tokens):
    n = len(parent)
    choice = [int(np.flatnonzero(r == r.max())[0]) for r in rows]
    ok = [True] + [False] * (n - 1)
    for i in range(1, n):                       # parents come first
        ok[i] = ok[parent[i]] and tokens[i] == choice[parent[i]]
    nodes = [i for i in range(n) if ok[i]]
    depth = [0] * n
    for i in range(1, n):
        depth[i] = depth[parent[i]] + 1
    nodes.sort(key=lambda i: depth[i])
    for x, y in zip(nodes, nodes[1:]):          # the consistent set is one path
        assert parent[y] == x
    last = nodes[-1]
    return dict(a=len(nodes) - 1, path=nodes, committed=[tokens[i] for i in nodes[1:]] + [choice[last]])


def pin_brute_force():
    rng = np.random.default_rng(12)
    for _ in range(400):
        n = int(rng.integers(1, 14))
        V = int(rng.integers(2, 5))
        parent, tokens = _random_tree(rng, n, V)
        if -1 in tokens[1:]:
            continue
        rows = rng.integers(0, 4, size=(n, V)).astype(float)
        assert ot.tree_walk_greedy(rows, parent, tokens) == _brute_force(rows, parent, tokens)


def pin_invalid_parent():
    rows = np.zeros((3, 4))
    for bad in ([-1, 0, 2], [-1, 1, 0], [-1, 0, -1], [-1, 0, 5]):
        try:
            ot.tree_walk_greedy(rows, bad, [0, 0, 0])
        except ValueError:
            continue
        raise AssertionError(f"parent list {bad} accepted")
    # and the batch form reports the request as -1 without touching its neighbours
    r = ot.tree_verify_batch(np.zeros((5, 4)), [-1, 0, 2, -1, 0], [0, 0, 0, 0, 0], [3, 2])
    assert r["accepted_len"].tolist() == [-1, 1]
    assert r["path_nodes"].tolist() == [-1, -1, -1, 0, 1]
    assert r["out_tokens"].tolist() == [-1, -1, -1, 0, 0]


TREE_PINS = [pin_golden_tree, pin_chain_is_linear_greedy, pin_brute_force, pin_invalid_parent]
