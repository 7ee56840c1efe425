"""Brute-force prefix attention, the definition the streaming oracle must reach.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

For every visit position t the partial output of the streaming method is, by
definition, softmax attention over exactly the tokens of the blocks visited so
far ("ART: Attention Run-time Termination ..." explainer, Technical Summary 2.1
and 2.4: streaming accumulation, permutation invariance of online softmax).
This module recomputes that from scratch for every t -- O(n^2) work, meant for
tiny inputs only -- on K/V given in logical (un-paged) token order.
"""

from __future__ import annotations

import math

import numpy as np


def prefix_attention_bruteforce(qv: np.ndarray, K_log: np.ndarray, V_log: np.ndarray, order, block_size: int,
                                seq_len: int) -> np.ndarray:
    """Return O[t] for t = 0..n-1: attention of ``qv`` over the tokens of blocks order[0..t].

    ``K_log``/``V_log`` are float64 [seq_len, D] in logical order.  Tokens at
    positions >= seq_len do not exist (the decode mask).
    """
    D = qv.shape[0]
    B = int(block_size)
    n = (int(seq_len) + B - 1) // B
    outs = np.zeros((n, D), dtype=np.float64)
    for t in range(n):
        pos = []
        for b in order[: t + 1]:
            lo = int(b) * B
            hi = min(lo + B, int(seq_len))
            pos.extend(range(lo, hi))
        idx = np.array(pos, dtype=np.int64)
        scores = np.array([float(np.dot(K_log[j], qv)) for j in idx]) / math.sqrt(D)
        mx = max(scores)
        w = np.array([math.exp(x - mx) for x in scores])
        outs[t] = (w[:, None] * V_log[idx]).sum(axis=0) / w.sum()
    return outs
