"""Pins of the oracle's input-contract check.

* hand-built tables whose first violation is worked out by hand (each code, the (sequence, position)
  precedence, the lowest code at one position, visit counts that hide a bad tail);
* every synthetic workload passes, and agrees with a second formulation of validity (the visited entries,
  sorted, are distinct and inside [0, n), the pages they name inside [0, num_pages));
* one planted corruption of a valid case is reported where it was planted.
"""

import numpy as np
import pytest

import oracle
from kv_cache_run_amd import synth, workloads as W

B = 16


def _tiny():
    # seq 0: 50 tokens -> 4 blocks; seq 1: 17 tokens -> 2 blocks; seq 2: 0 tokens
    table = np.array([[5, 6, 7, 8], [1, 2, 0, 0], [0, 0, 0, 0]], dtype=np.int32)
    order = np.array([[0, 3, 2, 1], [0, 1, -1, -1], [-1, -1, -1, -1]], dtype=np.int32)
    lens = np.array([50, 17, 0], dtype=np.int32)
    return table, order, lens


def _run(table, order, lens, visit=None, pages=9):
    return oracle.check_inputs(table, order, lens, num_pages=pages, block_size=B, visit_lens=visit)


def test_hand_built_cases():
    table, order, lens = _tiny()
    assert _run(table, order, lens) == (0, 0, 0, 0)
    # unused table cells and order entries past n_s are never looked at
    t2 = table.copy(); t2[1, 2:] = 99
    o2 = order.copy(); o2[1, 2:] = 77
    assert _run(t2, o2, lens) == (0, 0, 0, 0)
    # sequence length: negative, and one token past capacity (4 blocks of 16)
    l2 = lens.copy(); l2[1] = -1
    assert _run(table, order, l2) == (1, 1, 0, -1)
    l2 = lens.copy(); l2[2] = 65
    assert _run(table, order, l2) == (1, 2, 0, 65)
    # order entry outside [0, n): block 4 of a 4-block sequence at position 2
    o2 = order.copy(); o2[0, 2] = 4
    assert _run(table, o2, lens) == (2, 0, 2, 4)
    # repeated entry: positions 1 and 3 both hold block 3 -> the first of them
    o2 = order.copy(); o2[0, 3] = 3
    assert _run(table, o2, lens) == (3, 0, 1, 3)
    # page out of range for block 2 (visited at position 2), and negative for block 1 (position 3)
    t2 = table.copy(); t2[0, 2] = 9
    assert _run(t2, order, lens) == (4, 0, 2, 9)
    t2 = table.copy(); t2[0, 1] = -3
    assert _run(t2, order, lens) == (4, 0, 3, -3)
    # the earlier sequence wins over an earlier position of a later one
    o2 = order.copy(); o2[0, 3] = 2; o2[1, 0] = 5
    assert _run(table, o2, lens) == (3, 0, 2, 2)
    # at one position the lowest code wins: a repeated block whose page is also bad
    o2 = order.copy(); o2[0, 3] = 2
    t2 = table.copy(); t2[0, 2] = 100
    assert _run(t2, o2, lens) == (3, 0, 2, 2)
    # visit counts: a bad tail past visit_lens is not visited; counts clamp to [0, n]
    o2 = order.copy(); o2[0, 3] = 0
    assert _run(table, o2, lens) == (3, 0, 0, 0)
    assert _run(table, o2, lens, visit=np.array([3, 2, 0])) == (0, 0, 0, 0)
    assert _run(table, o2, lens, visit=np.array([-5, 2, 9])) == (0, 0, 0, 0)
    assert _run(table, o2, lens, visit=np.array([9, 2, 0])) == (3, 0, 0, 0)
    # a visited subset need not hold every block, only distinct ones
    o2 = order.copy(); o2[0, :2] = [3, 1]
    assert _run(table, o2, lens, visit=np.array([2, 2, 0])) == (0, 0, 0, 0)


def test_full_capacity_length_and_its_order():
    table, order, lens = _tiny()
    # 64 tokens fill the 4 blocks exactly: still valid
    assert _run(table, order, np.array([64, 17, 0], dtype=np.int32)) == (0, 0, 0, 0)


def _valid_by_sorting(case, pages):
    bt, bo, sl = case["block_table"], case["block_order"], case["seq_lens"]
    vl = case.get("visit_lens")
    for s in range(bo.shape[0]):
        L = int(sl[s])
        if not 0 <= L <= bo.shape[1] * case["block_size"]:
            return False
        n = -(-L // case["block_size"])
        v = n if vl is None else min(max(int(vl[s]), 0), n)
        e = np.sort(bo[s, :v])
        if v and (e[0] < 0 or e[-1] >= n or np.any(e[1:] == e[:-1])):
            return False
        if v and not np.all((bt[s, e] >= 0) & (bt[s, e] < pages)):
            return False
    return True


@pytest.mark.parametrize("w", [W.TINY, W.LLAMA3_8B, W.RAGGED, W.QWEN_FP8])
def test_workloads_pass_and_planted_corruptions_are_found(w):
    kw = {} if isinstance(w.context, tuple) else dict(context=min(w.context, 3000))  # ragged: its own lengths
    case = synth.make_case(w, batch=3, **kw)
    pages = case["k_pages"].shape[0]
    args = (case["block_table"], case["block_order"], case["seq_lens"])
    assert oracle.check_inputs(*args, num_pages=pages, block_size=case["block_size"]) == (0, 0, 0, 0)
    assert _valid_by_sorting(case, pages)
    rng = np.random.default_rng(5)
    n = -(-case["seq_lens"].astype(np.int64) // case["block_size"])
    for trial in range(6):
        s = int(rng.integers(0, 3))
        if n[s] < 3:
            continue
        t, u = sorted(int(x) for x in rng.choice(n[s], size=2, replace=False))
        kind = trial % 3
        bo, bt = case["block_order"].copy(), case["block_table"].copy()
        if kind == 0:
            bo[s, u] = n[s] + 3
            want = (2, s, u, int(n[s] + 3))
        elif kind == 1:
            bo[s, u] = bo[s, t]
            want = (3, s, t, int(bo[s, t]))
        else:
            bt[s, bo[s, u]] = pages
            want = (4, s, u, pages)
        got = oracle.check_inputs(bt, bo, case["seq_lens"], num_pages=pages, block_size=case["block_size"])
        assert got == want, (trial, got, want)
        bad = dict(case, block_order=bo, block_table=bt)
        assert not _valid_by_sorting(bad, pages)
