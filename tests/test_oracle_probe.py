"""Pins of the oracle's probe-vector detector (the statistics over a subset of the output's coordinates; the ART
explainer's Technical Summary 2.2 mentions monitoring such a subset).

The scores do not depend on V, so the coordinates idx of the streaming output are exactly those of the same
attention with every other value column set to zero, whose remaining output coordinates are exactly 0 and add
nothing to norms or inner products.  Hence, independently of the oracle's probe code:

* the probe over idx stops where the plain detector stops on the cache whose V is zero outside the columns idx;
* the probe over every coordinate is the plain detector;
* the output at the stop is the whole-vector attention output over the folded blocks.
"""

import numpy as np
import pytest

import oracle
from tests.helpers import build_case, oarr, okw


def _logical(seed, Hq=4, Hkv=2, D=32, B=4, L=120):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, Hq, D))
    K = rng.standard_normal((1, Hkv, L, D))
    V = rng.standard_normal((1, Hkv, L, D))
    g = Hq // Hkv
    for k in range(Hkv):
        qb = q[0, k * g:(k + 1) * g].sum(0)
        pos = rng.choice(L, size=L // 8, replace=False)
        K[0, k, pos] = 6.0 * qb / np.linalg.norm(qb)
    return q, K, V, B


@pytest.mark.parametrize("idx", [np.arange(8), np.arange(16), np.arange(0, 32, 4), np.array([3, 17, 30])],
                         ids=["lead8", "lead16", "every4", "scattered3"])
def test_probe_equals_plain_detector_on_restricted_values(idx):
    q, K, V, B = _logical(1)
    case = build_case(q, K, V, B)
    Vz = np.zeros_like(V)
    Vz[..., idx] = V[..., idx]
    restricted = build_case(q, K, Vz, B)
    for em, ed, p in [(1e-2, 1e-3, 2), (3e-2, 1e-2, 1), (1e-3, 1e-4, 3)]:
        a = oracle.art_reference(*oarr(case), eps_mag=em, eps_dir=ed, patience=p, probe=idx, **okw(case))
        b = oracle.art_reference(*oarr(restricted), eps_mag=em, eps_dir=ed, patience=p, **okw(restricted))
        assert np.array_equal(a["stop"], b["stop"]), (em, ed, p)
        assert np.allclose(a["out"][..., idx], b["out"][..., idx], rtol=1e-12, atol=1e-14)


def test_probe_of_every_coordinate_is_the_plain_detector():
    q, K, V, B = _logical(2)
    case = build_case(q, K, V, B)
    a = oracle.art_reference(*oarr(case), eps_mag=1e-2, eps_dir=1e-3, patience=2, probe=np.arange(32), **okw(case))
    b = oracle.art_reference(*oarr(case), eps_mag=1e-2, eps_dir=1e-3, patience=2, **okw(case))
    assert np.array_equal(a["stop"], b["stop"]) and np.array_equal(a["out"], b["out"])


def test_output_at_a_probe_stop_is_the_whole_vector():
    q, K, V, B = _logical(3)
    case = build_case(q, K, V, B)
    r = oracle.art_reference(*oarr(case), eps_mag=3e-2, eps_dir=1e-2, patience=1, probe=np.arange(4), **okw(case))
    for h in range(4):
        st = int(r["stop"][0, h])
        ref = oracle.prefix_output(*oarr(case), s=0, h=h, nfold=st, **okw(case))
        assert np.allclose(r["out"][0, h], ref, rtol=1e-12, atol=1e-14)
