"""Plain fp64 CPU oracle for the verification step of one speculative-decoding round.

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and the cpu_baseline
leg of bench.py may import or run anything in oracle/.  The product path (the
HIP library and its Python binding) never calls it and shares no code with it.

What is computed, and where the pages define it
-----------------------------------------------
Pages cited:
  [CZ]   chzhyang, "Speculative Decoding: Medusa, MTP, EAGLE, DFlash, DDTree, and DSpark"
  [VLLM] vLLM blog post "speculative-decoding-amd-gpus" (2026-08-20)
  [HN]   Hacker News Chinese digest of the vLLM post

* Verification runs left to right; at the first rejection the round is cut and
  every later draft token is discarded ([VLLM] "Core idea of speculative
  decoding"; [CZ] section 1, the A B C D -> A B R example).
* Stochastic rows: p_i is the target distribution, q_i the proposal actually
  sampled from; draft y_i is kept with probability min(1, p_i(y_i)/q_i(y_i))
  ([CZ] section 1, equation for alpha_i).
* At the first rejection the correction is drawn from the normalised positive
  residual [p_i - q_i]_+; when every draft survives, one more token is drawn
  from the target ([CZ] section 1, paragraph after the alpha equation).
* Greedy rows: a draft survives while it equals the target's argmax; the
  target's choice replaces the first mismatch ([CZ] section 1 "Greedy
  equivalence"; [VLLM] "A simple accept/reject example").
* Temperature is applied to target and draft alike ([CZ] section 1, last
  paragraph: temperature must be incorporated consistently).
* The accepted length excludes the correction/bonus token ([CZ] section 2,
  definition of A).

Readings taken where the pages leave a step open:
  R1  p = softmax(z / T), q = softmax(d / T), the same fp32 temperature T for
      both, widened exactly to fp64.
  R2  Greedy ignores T and takes the lowest token id among tied maxima.
  R3  With u uniform on [0, 1): keep y iff u * q(y) < p(y).  This is the
      min(1, p/q) rule without a division; q(y) = 0 keeps iff p(y) > 0.
  R4  One uniform per draft position (u_accept) and one per request for the
      single final draw, correction or bonus (u_final = w).
  R5  Inverse CDF in ascending token id: t = min{t : C_t > w * Z} with C_t the
      running fp64 sum; if rounding leaves no such t, the last id with
      positive weight.
  R6  A residual whose total is exactly 0 (p == q numerically) falls back to
      drawing from p.
  R7  Each request has k_b >= 0 drafts and k_b + 1 target rows; k_b = 0 just
      draws the bonus (stochastic) or takes the argmax (greedy).
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

ORACLE_IS_TEST_INFRASTRUCTURE = True


def widen_temperature(T) -> float:
    """R1: the fp32 temperature the kernels see, as an exact fp64 value."""
    return float(np.float32(T))


def tempered_softmax(logits, T: float) -> np.ndarray:
    """p = exp((z - max z)/T) / sum, in fp64 ([CZ] section 1: p_i, q_i; reading R1)."""
    z = np.asarray(logits, dtype=np.float64)
    e = np.exp((z - z.max()) / T)
    return e / e.sum()


def lowest_argmax(logits) -> int:
    """Greedy target choice: lowest id attaining the row maximum (reading R2)."""
    z = np.asarray(logits, dtype=np.float64)
    return int(np.flatnonzero(z == z.max())[0])


def keeps_draft(u: float, p_y: float, q_y: float) -> bool:
    """Ratio test of [CZ] section 1 (alpha_i = min(1, p/q)), in the form of reading R3."""
    return float(u) * q_y < p_y


def accept_margin(u: float, p_y: float, q_y: float) -> float:
    """Relative distance of the ratio test u * q(y) < p(y) from its boundary:
    |u q(y) - p(y)| / max(u q(y), p(y)); 1 when both sides are 0 (decided
    exactly).  A mismatch on a test closer than 1e-6 is a near-tie."""
    a, b = float(u) * q_y, p_y
    top = max(a, b)
    return 1.0 if top == 0.0 else abs(a - b) / top


def positive_residual(p: np.ndarray, q: np.ndarray) -> np.ndarray:
    """[p - q]_+ elementwise ([CZ] section 1, correction after the first rejection)."""
    return np.maximum(p - q, 0.0)


def inverse_cdf(weights: np.ndarray, w: float):
    """Draw with one uniform w from unnormalised `weights` (reading R5).

    Returns (token, total, margin).  The margin is the distance of w * total
    from the nearer edge of the chosen token's cumulative interval
    [C_(t-1), C_t], relative to the total, so it does not depend on the scale
    of the weights (a residual [p - q]_+ of total 1e-9 and one of total 0.5
    with the same shape have the same margin).
    """
    c = np.cumsum(np.asarray(weights, dtype=np.float64))   # sequential, ascending id
    total = float(c[-1])
    thr = float(w) * total
    hits = np.flatnonzero(c > thr)
    if hits.size:
        t = int(hits[0])
    else:
        t = int(np.flatnonzero(weights > 0)[-1])
    lo = float(c[t - 1]) if t > 0 else 0.0
    margin = min(abs(lo - thr), abs(float(c[t]) - thr)) / total if total > 0 else 0.0
    return t, total, margin


def verify_request(target_rows: np.ndarray, draft_rows: Optional[np.ndarray],
                   tokens: np.ndarray, greedy: bool, T: Optional[float],
                   u_accept: np.ndarray, w: float, early_exit: bool = False) -> dict:
    """One request: k drafts, k+1 target rows, left-to-right verification.

    Returns accepted length a (excludes the final token), the committed tokens
    (a drafts + the correction or bonus), p(y_i) / q(y_i) for every draft row
    (stochastic requests; -1 for greedy ones), the residual mass Z (-1 when the
    bonus was drawn or the request is greedy) and the smallest decision margin
    (over the ratio tests up to the cut and the final draw).

    early_exit: compute the distributions of a position only when its test is
    reached (drafts after the first rejection are discarded unread, [VLLM]
    "Core idea of speculative decoding"); p(y_i), q(y_i) are then -1 after
    the cut, everything else is the same.
    """
    k = int(len(tokens))
    assert target_rows.shape[0] == k + 1
    p_y = np.full(k, -1.0)
    q_y = np.full(k, -1.0)
    if greedy:
        for i in range(k):
            g = lowest_argmax(target_rows[i])
            if int(tokens[i]) != g:
                return dict(a=i, committed=[int(x) for x in tokens[:i]] + [g],
                            p_y=p_y, q_y=q_y, resid_mass=-1.0, margin=math.inf)
        g = lowest_argmax(target_rows[k])
        return dict(a=k, committed=[int(x) for x in tokens] + [g],
                    p_y=p_y, q_y=q_y, resid_mass=-1.0, margin=math.inf)

    T = widen_temperature(T)
    V = target_rows.shape[1]
    for y in tokens:
        if not (0 <= int(y) < V):
            raise ValueError(f"draft token {int(y)} outside [0, {V})")
    ps, qs = {}, {}

    def dists(i):
        """p_i, q_i of position i (computed once), with p(y_i), q(y_i)."""
        if i not in ps:
            ps[i] = tempered_softmax(target_rows[i], T)
            qs[i] = tempered_softmax(draft_rows[i], T)
            p_y[i] = ps[i][int(tokens[i])]
            q_y[i] = qs[i][int(tokens[i])]
        return ps[i], qs[i]

    if not early_exit:
        for i in range(k):
            dists(i)
    margin = math.inf
    for i in range(k):
        p_i, q_i = dists(i)
        margin = min(margin, accept_margin(u_accept[i], p_y[i], q_y[i]))
        if not keeps_draft(u_accept[i], p_y[i], q_y[i]):
            r = positive_residual(p_i, q_i)
            if float(np.cumsum(r)[-1]) > 0.0:
                t, Z, m = inverse_cdf(r, w)
            else:                                   # reading R6
                t, _, m = inverse_cdf(p_i, w)
                Z = 0.0
            return dict(a=i, committed=[int(x) for x in tokens[:i]] + [t],
                        p_y=p_y, q_y=q_y, resid_mass=Z, margin=min(margin, m))
    p_bonus = tempered_softmax(target_rows[k], T)
    t, _, m = inverse_cdf(p_bonus, w)
    return dict(a=k, committed=[int(x) for x in tokens] + [t],
                p_y=p_y, q_y=q_y, resid_mass=-1.0, margin=min(margin, m))


def verify_batch(target, draft, tokens, num_draft, greedy, temperature,
                 u_accept, u_final, early_exit: bool = False) -> dict:
    """A packed batch (layout of the C ABI) -> per-request results.

    target: [K+B, V], row of (b, i) = off[b] + b + i;  draft: [K, V] or None,
    row of (b, i) = off[b] + i;  tokens, u_accept: [K];  u_final, greedy: [B].
    Output arrays follow the C ABI: out_tokens [K+B] with -1 in unused slots.
    """
    num_draft = np.asarray(num_draft, dtype=np.int64)
    B = num_draft.shape[0]
    K = int(num_draft.sum())
    off = np.concatenate([[0], np.cumsum(num_draft)])
    greedy = np.ones(B, bool) if greedy is None else np.asarray(greedy, bool)
    acc = np.zeros(B, np.int64)
    out = np.full(K + B, -1, np.int64)
    p_y = np.full(K, -1.0)
    q_y = np.full(K, -1.0)
    resid = np.full(B, -1.0)
    margin = np.full(B, math.inf)
    for b in range(B):
        k = int(num_draft[b])
        t0 = int(off[b]) + b
        d0 = int(off[b])
        res = verify_request(
            np.asarray(target[t0:t0 + k + 1]),
            None if greedy[b] else np.asarray(draft[d0:d0 + k]),
            np.asarray(tokens[d0:d0 + k]), bool(greedy[b]), temperature,
            np.asarray(u_accept[d0:d0 + k]), float(u_final[b]), early_exit)
        acc[b] = res["a"]
        out[t0:t0 + len(res["committed"])] = res["committed"]
        p_y[d0:d0 + k] = res["p_y"]
        q_y[d0:d0 + k] = res["q_y"]
        resid[b] = res["resid_mass"]
        margin[b] = res["margin"]
    return dict(accepted_len=acc, out_tokens=out, p_draft=p_y, q_draft=q_y,
                resid_mass=resid, margin=margin)
