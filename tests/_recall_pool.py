"""Worker for the peaked-attention recall test: the oracle's recall figures of
one (batch, head) problem, computed in a separate CPU process (numpy and the
oracle only, no GPU), so that every problem of the workload can be measured
on the host's cores while the test holds the GPU."""
import numpy as np

import oracle as O


def problem_recall(args):
    """args = (x [L, D] float64, queries, {n_h: (sorted_idx, undo_idx)}, chunk_len).
    Returns per round count: R@1, R@16, attention mass, the mean size of the
    query's window union, and per query the bracket test of the mass; plus the
    number of queries whose 2-round windows are contained in their 8-round
    windows (all but those in round 0's first chunk, whose look-back differs)."""
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):  # one BLAS thread per worker process
        return _problem_recall(args)


def _problem_recall(args):
    x, q, perms, C = args
    L = x.shape[0]
    out = {}
    for n_h, (s, u) in perms.items():
        unions = [len(O.attended_positions(s, u, C, int(i))) for i in q]
        mass_lo = mass_hi = 0.0
        for i, n in zip(q, unions):
            # On (nearly) unit vectors every logit lies within |x_i|/8 of 0, so
            # each exact weight is within a factor e^{+-|x_i|/4} of 1/(L-1).
            r = float(np.linalg.norm(x[i])) / 4.0
            mass_lo += (n - 1) * np.exp(-r) / (L - 1)
            mass_hi += (n - 1) * np.exp(r) / (L - 1)
        out[n_h] = {
            "r1": O.recall_at_k(x, s, u, C, q, 1),
            "r16": O.recall_at_k(x, s, u, C, q, 16),
            "mass": O.attention_mass_recall(x, s, u, C, q),
            "mass_lo": mass_lo / len(q),
            "mass_hi": mass_hi / len(q),
            "chance": float(np.mean([(n - 1) / (L - 1) for n in unions])),
        }
    contained = eligible = 0
    if 2 in perms and 8 in perms:
        (s2, u2), (s8, u8) = perms[2], perms[8]
        for i in q:
            if u2[0, i] < C:
                continue
            eligible += 1
            contained += int(O.attended_positions(s2, u2, C, int(i)) <= O.attended_positions(s8, u8, C, int(i)))
    out["contained"] = (contained, eligible)
    return out
