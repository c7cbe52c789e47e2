"""Acceptance statistics of verification rounds (test infrastructure).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may use oracle/.

The signals are the ones the vLLM blog post "speculative-decoding-amd-gpus"
lists under "Monitor acceptance behavior" and tabulates in its Appendix:
mean accepted length, overall acceptance rate and per-position acceptance.
chzhyang, "Speculative Decoding: ...", section 10 (item 5) asks to state
whether they count the bonus token; here:

  mean_accepted  = sum a_b / n                      (drafts kept, no final token)
  mal            = 1 + mean_accepted                (counts the correction/bonus token)
  ar             = sum a_b / sum k_b                (kept drafts over proposed drafts)
  per_position j = #{b : a_b >= j} / #{b : k_b >= j},  j = 1..max_pos

Requests whose accepted length is negative (invalid input) are not counted.
With every k_b = N these give the Appendix identities mal = 1 + sum_j p_j and
ar = (mal - 1) / N.
"""
from __future__ import annotations

import numpy as np


def acceptance_stats(accepted_len, num_draft, max_pos: int) -> dict:
    a = np.asarray(accepted_len, dtype=np.int64)
    k = np.asarray(num_draft, dtype=np.int64)
    ok = a >= 0
    a, k = a[ok], k[ok]
    n = int(a.size)
    sa, sk = int(a.sum()), int(k.sum())
    mean = sa / n if n else -1.0
    per = np.full(max_pos, -1.0)
    for j in range(1, max_pos + 1):
        proposed = int((k >= j).sum())
        if proposed:
            per[j - 1] = int((a >= j).sum()) / proposed
    return dict(rounds=n, mean_accepted=mean, mal=(1.0 + mean) if n else -1.0,
                ar=(sa / sk) if sk else -1.0, per_position=per)
