"""CPU oracle (test infrastructure only): a plain float64 implementation of the
shared-QK LSH-attention forward pass (lsh_oracle) and its gradient
(lsh_backward, float64 autograd), used to check the HIP path."""
from .lsh_oracle import *  # noqa: F401,F403
from .lsh_oracle import (SELF_LOGIT, attended_positions, attention_mass_recall, chunk_attention,  # noqa: F401
                         forward, forward_problem, full_attention, hash_buckets, recall_at_k,
                         sort_by_bucket, token_output, unsort_combine, window_slots)
