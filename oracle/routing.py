"""Top-k expert routing that lays out the grouped (MoE) GEMM inputs.

TEST INFRASTRUCTURE ONLY (see the package docstring).

DeepSeek is a mixture-of-experts model (page 4 section 1.2 names the MoE
structure); the pages give no router.  Reading used here: every token picks
the k experts with the largest raw router logits (a monotone gate such as
softmax or sigmoid picks the same set), ties going to the lower expert index,
with no group-limited routing.  The (expert, token) pairs are then ordered by
expert and, within an expert, by token; offsets[e] is the exclusive prefix sum
of the per-expert counts.
"""

import numpy as np


def topk_route(logits, k):
    """logits [T, E] -> (rows int64 [T*k], experts int64 [T*k], offsets int64 [E+1]).

    rows[i] is the token of the i-th expert-sorted pair, experts[i] its expert.
    """
    logits = np.asarray(logits)
    T, E = logits.shape
    picks = np.empty((T, k), np.int64)
    for t in range(T):
        # stable sort of the negated logits: equal logits keep index order
        order = np.argsort(-logits[t].astype(np.float64), kind="stable")
        picks[t] = order[:k]
    tok = np.repeat(np.arange(T, dtype=np.int64), k)
    exp = picks.reshape(-1)
    order = np.lexsort((tok, exp))            # primary key expert, then token
    counts = np.bincount(exp, minlength=E)
    offsets = np.zeros(E + 1, np.int64)
    offsets[1:] = np.cumsum(counts)
    return tok[order], exp[order], offsets
