"""The decode's input contract, checked by plain loops (TEST INFRASTRUCTURE ONLY; see art_oracle.py's header).

The ART explainer (Technical Summary 2.4) has the decode walk a sequence's KV blocks in a traversal order
(block 0, the attention sink, among them) through a paged cache.  The decode takes as given what that
needs of its integer inputs; this module states it, position by position:

* ``seq_lens[s]`` lies in [0, max_blocks * block_size]; then n_s = ceil(seq_lens[s] / block_size);
* the visited positions are t < v_s, v_s = n_s, or ``visit_lens[s]`` clamped to [0, n_s];
* at a visited position, the order entry b = ``block_order[s][t]`` lies in [0, n_s), no other visited
  position of the row holds the same b, and the page ``block_table[s][b]`` lies in [0, num_pages).

The first violation in (sequence, visit position) order is reported, and at one position the lowest code:
1 sequence length out of range (position 0), 2 order entry out of range, 3 order entry repeated,
4 page out of range.
"""

from __future__ import annotations

from collections import Counter
from typing import Tuple

import numpy as np

OK, SEQ_LEN, ORDER_RANGE, ORDER_REPEAT, PAGE_RANGE = 0, 1, 2, 3, 4


def check_inputs(block_table, block_order, seq_lens, *, num_pages: int, block_size: int,
                 visit_lens=None) -> Tuple[int, int, int, int]:
    """(code, sequence, visit position, offending value) of the first violation, or (0, 0, 0, 0).

    The value is seq_lens[s] for code 1, the order entry for codes 2 and 3, the page for code 4."""
    block_table = np.asarray(block_table)
    block_order = np.asarray(block_order)
    batch, max_blocks = block_order.shape
    for s in range(batch):
        L = int(seq_lens[s])
        if L < 0 or L > max_blocks * block_size:
            return SEQ_LEN, s, 0, L
        n = -(-L // block_size)
        v = n if visit_lens is None else min(max(int(visit_lens[s]), 0), n)
        row = [int(x) for x in block_order[s, :v]]
        times = Counter(row)  # how often each entry occurs among the visited positions
        for t, b in enumerate(row):
            if not 0 <= b < n:
                return ORDER_RANGE, s, t, b
            if times[b] > 1:
                return ORDER_REPEAT, s, t, b
            pg = int(block_table[s, b])
            if not 0 <= pg < num_pages:
                return PAGE_RANGE, s, t, pg
    return OK, 0, 0, 0
