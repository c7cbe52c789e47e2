"""fp64 CPU oracle for one round of draft-token verification.

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import it.  Shares no code with the HIP path.
"""
from .verify import (verify_batch, verify_request, tempered_softmax, lowest_argmax,
                     keeps_draft, positive_residual, inverse_cdf, widen_temperature)
from .cost_model import time_per_token, expected_progress
from .tree import tree_walk_greedy, tree_verify_batch
from .adaptive import progress_table, choose_length, adaptive_batch

__all__ = ["verify_batch", "verify_request", "tempered_softmax", "lowest_argmax",
           "keeps_draft", "positive_residual", "inverse_cdf", "widen_temperature",
           "time_per_token", "expected_progress", "tree_walk_greedy", "tree_verify_batch",
           "progress_table", "choose_length", "adaptive_batch"]
