"""Plain CPU oracle for confidence-driven verification length (DSpark) and the
compaction of the chosen windows into a packed ragged batch.

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and the cpu_baseline
leg of bench.py may import or run anything in oracle/.  The product path never
calls it and shares no code with it.

What is computed, and where the pages define it
-----------------------------------------------
[CZ] chzhyang, "Speculative Decoding: Medusa, MTP, EAGLE, DFlash, DDTree, and
DSpark":
* section 5 DSpark: with conditional confidences c_i, the estimated chance of
  accepting through position j is s_j = c_1 c_2 ... c_j, and verifying a
  prefix of length k has estimated progress 1 + s_1 + ... + s_k; a scheduler
  asks whether one more position is worth its marginal cost, and only a
  compact, variable-length verification (windows packed back to back) turns a
  shorter window into less work;
* section 2: a round costs T_draft + T_verify + T_overhead and advances
  E[A] + 1 tokens, so the time per token is cost / progress;
* section 9: the cost of each window length comes from a table profiled for
  the deployment.

Readings taken where the pages leave a step open:
  D1  Each request chooses its own length k in 0..N from one table cost[0..N]
      of positive costs (the cost of a round whose window has k positions),
      maximising progress(k) / cost[k] (equivalently minimising the time per
      token of section 2).  Ties go to the smallest k.
  D2  Arithmetic in fp64 in this order: s_0 = 1; for j = 1..k: s_j = s_{j-1} *
      c_j (c_j an fp32 input widened exactly); progress(k) = 1 + s_1 + ... +
      s_k summed left to right; ratio(k) = progress(k) / cost[k], correctly
      rounded.  A decision taken in floating point is taken in this precision
      on both sides.
  D3  The kept window of request b is its first k_b drafts; the packed batch
      lists the kept drafts request after request (offsets = exclusive prefix
      sums of k), with src_index = b * N + i naming the position each kept
      draft came from in the [B][N] input block.
"""
from __future__ import annotations

import numpy as np

ORACLE_IS_TEST_INFRASTRUCTURE = True


def progress_table(conf) -> np.ndarray:
    """progress(k) for k = 0..N (section 5 DSpark; reading D2)."""
    out = [1.0]
    s = 1.0
    total = 1.0
    for c in conf:
        s = s * float(np.float32(c))
        total = total + s
        out.append(total)
    return np.array(out)


def choose_length(conf, cost) -> tuple:
    """Reading D1: k maximising progress(k) / cost[k], smallest k on ties.
    Returns (k, progress(k))."""
    prog = progress_table(conf)
    best_k, best_r = 0, None
    for k in range(len(prog)):
        r = prog[k] / float(cost[k])
        if best_r is None or r > best_r:
            best_k, best_r = k, r
    return best_k, float(prog[best_k])


def adaptive_batch(conf, cost, tokens) -> dict:
    """Per-request choice, then the packed ragged batch (reading D3).

    conf: [B, N] confidences; cost: [N + 1]; tokens: [B, N] drafted tokens.
    Returns num_draft [B], offsets [B + 1], tokens [K'], src_index [K'],
    progress [B].
    """
    conf = np.asarray(conf)
    tokens = np.asarray(tokens)
    B, N = conf.shape
    if len(cost) != N + 1:
        raise ValueError("cost table needs N + 1 entries")
    if not all(float(c) > 0.0 for c in cost):
        raise ValueError("costs must be positive")
    ks = np.zeros(B, np.int64)
    prog = np.zeros(B)
    for b in range(B):
        ks[b], prog[b] = choose_length(conf[b], cost)
    offsets = np.concatenate([[0], np.cumsum(ks)]).astype(np.int64)
    src = np.concatenate([b * N + np.arange(ks[b]) for b in range(B)]).astype(np.int64) \
        if B else np.zeros(0, np.int64)
    toks = tokens.reshape(-1)[src] if src.size else np.zeros(0, np.int64)
    return dict(num_draft=ks, offsets=offsets, tokens=toks.astype(np.int64), src_index=src,
                progress=prog)
