"""Pins of the oracle for ART over a pruned cache (visit_lens: only the first visit_lens[s] entries of the
order are visited).  The ART explainer (Technical Summary 2.4) layers ART over cache-pruning methods through
the traversal order, so the rule over a subset must be the rule over a cache that holds only that subset:

* visit_lens = n is the plain call;
* the oracle with visit_lens equals the plain oracle on a *compacted* cache built independently here (the
  visited blocks only, renumbered in logical order, block 0 kept as block 0 and a partial last block kept
  last): the same stops and outputs, ART and full attention;
* a subset without block 0 never stops early (the block-0 condition never holds): stop = visit_lens;
* an empty subset gives out = 0, stop = 0.
"""

import math

import numpy as np
import pytest

import oracle
from tests.helpers import build_case, oarr, okw


def _logical(seed, Hq=4, Hkv=2, D=16, B=4, L=90):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, Hq, D))
    K = rng.standard_normal((1, Hkv, L, D))
    V = rng.standard_normal((1, Hkv, L, D))
    g = Hq // Hkv
    for k in range(Hkv):
        qb = q[0, k * g:(k + 1) * g].sum(0)
        pos = rng.choice(L, size=L // 10, replace=False)
        K[0, k, pos] = 6.0 * qb / np.linalg.norm(qb)
    return q, K, V, B, L


def _compact(q, K, V, B, L, order):
    """A cache holding only the visited blocks (in ``order``), renumbered in logical order."""
    n = (L + B - 1) // B
    S = sorted(int(b) for b in order)
    rank = {b: i for i, b in enumerate(S)}
    rows = np.concatenate([np.arange(b * B, min((b + 1) * B, L)) for b in S])
    Kc, Vc = K[:, :, rows], V[:, :, rows]
    Lc = len(rows)
    assert S[-1] == n - 1 or Lc == len(S) * B  # a partial block can only be the last one
    return build_case(q, Kc, Vc, B, seq_lens=[Lc], order=[[rank[int(b)] for b in order]], page_seed=5)


def _art(case, em, ed, p, vl=None):
    return oracle.art_reference(*oarr(case), eps_mag=em, eps_dir=ed, patience=p, visit_lens=vl, **okw(case))


def test_visiting_every_block_is_the_plain_call():
    q, K, V, B, L = _logical(0)
    case = build_case(q, K, V, B)
    n = (L + B - 1) // B
    a = _art(case, 1e-2, 1e-3, 2)
    b = _art(case, 1e-2, 1e-3, 2, vl=np.array([n]))
    assert np.array_equal(a["stop"], b["stop"]) and np.array_equal(a["out"], b["out"])


@pytest.mark.parametrize("seed", [1, 2, 3, 4])
def test_pruned_call_equals_the_compacted_cache(seed):
    q, K, V, B, L = _logical(seed)
    n = (L + B - 1) // B
    rng = np.random.default_rng(100 + seed)
    if seed == 1:   # block 0 plus a recent window, newest first (the default order's head)
        order = [0] + list(range(n - 1, n - 9, -1))
    else:           # a random subset holding block 0 (and, for seed 3, the partial last block), random order
        rest = rng.choice(np.arange(1, n - 1), size=int(rng.integers(3, n - 3)), replace=False).tolist()
        order = [0] + rest + ([n - 1] if seed == 3 else [])
        order = [order[i] for i in rng.permutation(len(order))]
    full_order = order + [b for b in range(n) if b not in order]
    case = build_case(q, K, V, B, order=[full_order])
    comp = _compact(q, K, V, B, L, order)
    for em, ed, p in [(1e-2, 1e-3, 2), (5e-2, 1e-2, 1), (1e-3, 1e-4, 3)]:
        a = _art(case, em, ed, p, vl=np.array([len(order)]))
        b = _art(comp, em, ed, p)
        assert np.array_equal(a["stop"], b["stop"]), (em, ed, p)
        assert np.allclose(a["out"], b["out"], rtol=1e-12, atol=1e-14)
    fa = oracle.full_attention(case["q"], case["k_pages"], case["v_pages"], case["block_table"], case["seq_lens"],
                               block_order=case["block_order"], visit_lens=np.array([len(order)]), **okw(case))
    fb = oracle.full_attention(comp["q"], comp["k_pages"], comp["v_pages"], comp["block_table"], comp["seq_lens"],
                               **okw(comp))
    assert np.allclose(fa, fb, rtol=1e-12, atol=1e-14)


def test_subset_without_block_zero_never_stops_early():
    q, K, V, B, L = _logical(7)
    n = (L + B - 1) // B
    case = build_case(q, K, V, B, order=[list(range(n - 1, -1, -1))])  # block 0 visited last
    for vl in (1, 5, n - 1):
        r = _art(case, 10.0, 10.0, 1, vl=np.array([vl]))  # every test passes: only block 0 can hold it back
        assert np.all(r["stop"] == vl)
    r = _art(case, 10.0, 10.0, 1, vl=np.array([n]))
    assert np.all(r["stop"] == n)  # block 0 folded last, at position n - 1: the stop is n either way


def test_empty_subset():
    q, K, V, B, L = _logical(8)
    case = build_case(q, K, V, B)
    r = _art(case, 1e-2, 1e-3, 2, vl=np.array([0]))
    assert np.all(r["stop"] == 0) and np.all(r["out"] == 0.0)


def test_visits_must_be_distinct_blocks():
    q, K, V, B, L = _logical(9)
    case = build_case(q, K, V, B)
    bad = case["block_order"].copy()
    bad[0, 1] = bad[0, 0]
    with pytest.raises(ValueError):
        oracle.art_reference(*oarr(dict(case, block_order=bad)), eps_mag=1e-2, eps_dir=1e-3, patience=2,
                             visit_lens=np.array([3]), **okw(case))
