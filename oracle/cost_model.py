"""Round-level arithmetic the pages state in closed form (test infrastructure).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may use oracle/.
"""
from __future__ import annotations

from typing import Sequence


def time_per_token(t_draft: float, t_verify: float, t_overhead: float,
                   mean_accepted: float) -> float:
    """Steady-state cost per committed token: one round's expected time spread
    over E[A] + 1 tokens, A excluding the correction/bonus token
    (chzhyang, "Speculative Decoding: ...", section 2, equation for T_token)."""
    return (t_draft + t_verify + t_overhead) / (mean_accepted + 1.0)


def expected_progress(conf: Sequence[float], k: int) -> float:
    """Estimated progress of verifying a prefix of length k: 1 + sum_{j<=k} s_j with
    s_j = prod_{i<=j} c_i (chzhyang, section 5 DSpark, prefix-survival estimate)."""
    s, total = 1.0, 1.0
    for j in range(k):
        s *= float(conf[j])
        total += s
    return total
