"""Exhaustive pin of the patience/sink stop rule against an independent definition.

Independent definition (ART explainer, Technical Summary 2.3 and 2.4): the
head stops after the first visit position t at which the tests of the
``patience`` positions ending at t all passed (a test exists from position 1
on) and logical block 0 has been visited at some position <= t.  The stop
value is the number of folded blocks, t + 1; n when no position qualifies.
"""

import itertools

import numpy as np
import pytest

import oracle
from tests.helpers import build_case, oarr, okw


def _window_definition(passes, sink_pos, p):
    n = len(passes)
    for t in range(n):
        if t - p + 1 < 1:
            continue
        if sink_pos > t:
            continue
        if all(passes[u] for u in range(t - p + 1, t + 1)):
            return t + 1
    return n


@pytest.mark.parametrize("p", [1, 2, 3, 4, 5])
def test_stop_rule_exhaustive(p):
    for n in range(0, 13):
        for bits in itertools.product([False, True], repeat=max(n - 1, 0)):
            passes = [None] + list(bits) if n else []
            for sink_pos in sorted({0, 1, 3, n - 1} & set(range(n))) or [0]:
                sinks = [t == sink_pos for t in range(n)]
                want = _window_definition(passes, sink_pos, p) if n else 0
                assert oracle.stop_rule(passes, sinks, p) == want, (passes, sink_pos, p)


def test_stop_rule_rejects_bad_patience():
    with pytest.raises(ValueError):
        oracle.stop_rule([None, True], [True, False], 0)


@pytest.mark.parametrize("seed", range(6))
def test_streaming_loop_applies_the_same_rule_to_its_own_statistics(seed):
    """The per-head loop's stop equals stop_rule over its recorded test outcomes."""
    rng = np.random.default_rng(seed)
    D, B, n = 16, 4, 40
    q = rng.standard_normal((1, 2, D)).astype(np.float32)
    K = rng.standard_normal((1, 1, n * B, D)).astype(np.float32)
    heavy = rng.choice(n * B, size=12, replace=False)
    K[0, 0, heavy] = 3.0 * q[0, 0] / np.linalg.norm(q[0, 0])
    V = rng.standard_normal((1, 1, n * B, D)).astype(np.float32)
    order = [list(rng.permutation(n))]
    case = build_case(q, K, V, B, order=order, page_seed=seed)
    for eps_mag, eps_dir, p in [(2e-2, 2e-3, 2), (5e-2, 1e-2, 1), (1e-2, 1e-3, 3)]:
        for h in range(2):
            tr = oracle.head_stats_trajectory(*oarr(case), s=0, h=h, eps_mag=eps_mag, eps_dir=eps_dir, patience=p,
                                              **okw(case))
            passes = [None] + [bool(a < eps_mag and b < eps_dir) for a, b in zip(tr["d_mag"], tr["d_dir"])]
            assert tr["stop"] == oracle.stop_rule(passes, tr["sinks"], p)
            r = oracle.art_reference(*oarr(case), eps_mag=eps_mag, eps_dir=eps_dir, patience=p, **okw(case),
                                     pairs=[(0, h)])
            assert r["stop"][0, h] == tr["stop"]
