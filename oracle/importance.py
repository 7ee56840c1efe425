"""Importance-first visit order, plain float64 (TEST INFRASTRUCTURE ONLY; see art_oracle.py's header).

The ART explainer (Technical Summary 2.4) names "importance-first" beside "recency-first" as a traversal
order ART can run over; it does not define the importance.  The reading taken here:

* a block's key summary per kv-head is the mean of its valid key rows (what a cache could store when it
  writes the block);
* a block's score is the largest, over the query heads, of q_h . summary / sqrt(D) (a block matters when
  any head would attend to it);
* the order is block 0 first (the sink must be folded before any stop), then descending score, ties to the
  newer (higher) block, so equal scores reduce to recency-first.
"""

from __future__ import annotations

import math

import numpy as np

from .art_oracle import _decoder, _nblocks


def block_key_summary(k_pages, block_table, seq_lens, *, block_size: int, num_kv_heads: int, kv_dtype: str,
                      k_scale=None) -> np.ndarray:
    """float64 [num_pages, Hkv, D]: mean of each referenced block's valid key rows (NaN for other pages)."""
    dec = _decoder(kv_dtype)
    P, Hkv, B, D = k_pages.shape
    out = np.full((P, Hkv, D), np.nan)
    for s in range(block_table.shape[0]):
        L = int(seq_lens[s])
        for b in range(_nblocks(L, block_size)):
            pg = int(block_table[s, b])
            rows = min(block_size, L - b * block_size)
            for k in range(Hkv):
                K = dec(k_pages[pg, k, :rows])
                if kv_dtype == "fp8_e4m3fn":
                    K = K * float(k_scale[pg, k])
                out[pg, k] = K.mean(axis=0)
    return out


def block_scores(q, summary, block_table, seq_lens, *, block_size: int, num_kv_heads: int,
                 q_dtype: str) -> np.ndarray:
    """float64 [batch, max_blocks]: max over query heads of q_h . summary / sqrt(D) (NaN past n_s)."""
    Q = _decoder(q_dtype)(q)
    batch, Hq, D = Q.shape
    g = Hq // int(num_kv_heads)
    sc = np.full(block_table.shape, np.nan)
    for s in range(batch):
        for b in range(_nblocks(int(seq_lens[s]), block_size)):
            S = np.asarray(summary[int(block_table[s, b])], dtype=np.float64)
            sc[s, b] = max(float(Q[s, h] @ S[h // g]) for h in range(Hq)) / math.sqrt(D)
    return sc


def importance_order(scores: np.ndarray, seq_lens, *, block_size: int) -> np.ndarray:
    """int64 [batch, max_blocks] visit order (-1 past n_s): block 0, then descending score, ties newer first."""
    order = np.full(scores.shape, -1, dtype=np.int64)
    for s in range(scores.shape[0]):
        n = _nblocks(int(seq_lens[s]), block_size)
        if n == 0:
            continue
        rest = sorted(range(1, n), key=lambda b: (-scores[s, b], -b))
        order[s, :n] = [0] + rest
    return order
