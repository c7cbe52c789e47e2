"""Plain CPU oracle for greedy verification of a draft token tree (DDTree walk).

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and the cpu_baseline
leg of bench.py may import or run anything in oracle/.  The product path never
calls it and shares no code with it.

What is computed, and where the pages define it
-----------------------------------------------
[CZ] chzhyang, "Speculative Decoding: Medusa, MTP, EAGLE, DFlash, DDTree, and
DSpark", section 5 "DDTree: Build a Tree from Parallel Marginals":

* the drafted candidates form a tree; each node carries one token and sits at
  the position given by its depth, and the target scores every node with
  attention restricted to the node's ancestors, so the target row of a node is
  the target's next-token distribution after the node's prefix;
* verification walks down from the root following the target's selected token:
  while a child of the current node carries that token the walk moves to it;
  when no child does, the target's token is committed as the bonus token;
* only the accepted path survives (its nodes are the ones whose KV entries are
  kept).

Greedy selection is the target argmax, as for linear greedy verification ([CZ]
section 1 "Greedy equivalence"); the stochastic tree is out of scope (the pages
name it as needing its own procedure and do not give one).

Readings taken where the pages leave a step open:
  T1  Node 0 of every request is the root (the last committed token); its own
      token is not verified.  Every other node i has a parent p with
      0 <= p < i (nodes are listed parents first).  A parent outside that range
      makes the request invalid.
  T2  The target's choice is the lowest token id attaining the row maximum
      (reading R2 of the linear oracle).
  T3  If several children of the current node carry the chosen token (a tree a
      best-first search would not build), the walk follows the one with the
      lowest node index.
  T4  Outputs per request: a = accepted draft nodes; path = [0, n_1, ..., n_a],
      the node indices walked (root first); committed = the a accepted tokens
      followed by the bonus token (a + 1 tokens, as for the linear case).
"""
from __future__ import annotations

import numpy as np

from .verify import lowest_argmax

ORACLE_IS_TEST_INFRASTRUCTURE = True


def check_parents(parent) -> None:
    """Reading T1: 0 <= parent[i] < i for every non-root node."""
    for i in range(1, len(parent)):
        if not (0 <= int(parent[i]) < i):
            raise ValueError(f"node {i} has parent {int(parent[i])} outside [0, {i})")


def children_of(parent) -> list:
    """Children of every node in ascending node index (readings T1, T3)."""
    kids = [[] for _ in range(len(parent))]
    for i in range(1, len(parent)):
        kids[int(parent[i])].append(i)
    return kids


def tree_walk_greedy(target_rows, parent, tokens) -> dict:
    """[CZ] section 5: walk from the root along the target's selected tokens.

    target_rows: [n, V] target logits, row i = next-token logits after node i.
    parent, tokens: [n] (entry 0, the root's, is not used).
    Returns a (accepted draft nodes), path (node indices, root first) and
    committed (accepted tokens then the bonus token).
    """
    n = len(parent)
    if n < 1:
        raise ValueError("a tree has at least its root")
    check_parents(parent)
    kids = children_of(parent)
    path = [0]
    committed = []
    cur = 0
    while True:
        choice = lowest_argmax(target_rows[cur])
        follow = None
        for c in kids[cur]:                 # ascending index: reading T3
            if int(tokens[c]) == choice:
                follow = c
                break
        if follow is None:                  # no child carries it: the bonus token
            committed.append(choice)
            break
        committed.append(int(tokens[follow]))
        path.append(follow)
        cur = follow
    return dict(a=len(path) - 1, path=path, committed=committed)


def tree_verify_batch(target, parent, tokens, num_nodes) -> dict:
    """A packed batch of trees (layout of the C ABI) -> per-request results.

    Request b owns nodes noff[b] .. noff[b] + n_b - 1 (noff = exclusive prefix
    sum of num_nodes); parents are local indices.  Outputs follow the C ABI:
    accepted_len [B] (-1 for an invalid request), path_nodes [N] and
    out_tokens [N] with request b's entries from slot noff[b] on and -1 in
    every unused slot.
    """
    num_nodes = np.asarray(num_nodes, dtype=np.int64)
    B = num_nodes.shape[0]
    N = int(num_nodes.sum())
    noff = np.concatenate([[0], np.cumsum(num_nodes)])
    acc = np.full(B, -1, np.int64)
    path = np.full(N, -1, np.int64)
    out = np.full(N, -1, np.int64)
    for b in range(B):
        s, n = int(noff[b]), int(num_nodes[b])
        try:
            r = tree_walk_greedy(np.asarray(target[s:s + n]), np.asarray(parent[s:s + n]),
                                 np.asarray(tokens[s:s + n]))
        except ValueError:
            continue
        acc[b] = r["a"]
        path[s:s + len(r["path"])] = r["path"]
        out[s:s + len(r["committed"])] = r["committed"]
    return dict(accepted_len=acc, path_nodes=path, out_tokens=out)
