"""The stop-comparison rule: constructive check vs enumeration of every resolution."""

import itertools

import numpy as np
import pytest

import oracle
from oracle.feasible import AMBIG, FAIL, PASS


def _enumerate(status, sinks, p, n):
    amb = [i for i, s in enumerate(status) if s == AMBIG]
    stops = set()
    for bits in itertools.product([False, True], repeat=len(amb)):
        passes = [None] + [s == PASS for s in status]
        for i, b in zip(amb, bits):
            passes[i + 1] = b
        stops.add(oracle.stop_rule(passes, sinks, p))
    return stops


@pytest.mark.parametrize("seed", range(40))
def test_constructive_rule_equals_enumeration(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(2, 11))
    p = int(rng.integers(1, 4))
    status = rng.choice([PASS, FAIL, AMBIG], size=n - 1, p=[0.5, 0.3, 0.2])
    sink_pos = int(rng.integers(0, n))
    sinks = [t == sink_pos for t in range(n)]
    feasible = {s for s in range(n + 1) if oracle.feasible_stop(status, np.array(sinks), p, s, n)}
    assert feasible == _enumerate(list(status), sinks, p, n)


def test_classification_band():
    st = oracle.classify_tests(np.array([0.5e-3, 1e-3 - 2e-5, 1e-3 - 5e-6, 1e-3, 1e-3 + 2e-5, 0.0]),
                               np.array([0.0, 0.0, 0.0, 0.0, 0.0, 1e-4 + 5e-6]), 1e-3, 1e-4, band=1e-5)
    assert list(st) == [PASS, PASS, AMBIG, AMBIG, FAIL, AMBIG]
    # one definite failure decides the conjunction
    st = oracle.classify_tests(np.array([1e-3]), np.array([1.0]), 1e-3, 1e-4)
    assert list(st) == [FAIL]
