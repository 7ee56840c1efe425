"""Closed-form trajectories of the two statistics (hand-derived expected values).

With K = 0 every score is 0, so every valid token gets the same weight and the
partial output after t blocks is the plain mean of the V rows folded so far.
That makes O_t, both statistics and the stop position computable by hand.
The expected values live in ``tests/golden/closed_form.txt`` with their
derivations.
"""

import math
import os

import numpy as np
import pytest

import oracle
from tests.helpers import build_case, oarr, okw

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_form.txt")


def _golden():
    vals = {}
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, expr = line.split("=", 1)
            vals[key.strip()] = float(eval(expr, {"sqrt": math.sqrt, "__builtins__": {}}))  # noqa: S307
    return vals


G = _golden()


def _blocks_case(vblocks, D, B=4, order=None, K=None):
    """One sequence, one head; block b has all its V rows equal to vblocks[b]."""
    n = len(vblocks)
    V = np.concatenate([np.tile(np.asarray(v, np.float32), (B, 1)) for v in vblocks])[None, None]
    Kz = np.zeros_like(V) if K is None else K
    q = np.ones((1, 1, D), np.float32)
    od = (lambda m: range(m)) if order is None else [order]
    return build_case(q, Kz, V, B, order=od, page_seed=n)


def _traj(case, eps_mag=1e-3, eps_dir=1e-4, p=1):
    return oracle.head_stats_trajectory(*oarr(case), s=0, h=0, eps_mag=eps_mag, eps_dir=eps_dir, patience=p,
                                        **okw(case))


def test_constant_values_stop_after_patience_plus_one_blocks():
    rng = np.random.default_rng(0)
    D, B, n = 8, 4, 10
    c = rng.standard_normal(D).astype(np.float32)
    K = rng.standard_normal((1, 1, n * B, D)).astype(np.float32)
    case = _blocks_case([c] * n, D, B, K=K)
    for p in (1, 2, 3, 5):
        r = oracle.art_reference(*oarr(case), eps_mag=1e-12, eps_dir=1e-12, patience=p, **okw(case))
        assert r["stop"][0, 0] == p + 1
        assert np.allclose(r["out"][0, 0], c, rtol=1e-12)
    tr = _traj(case)
    assert np.all(tr["d_mag"] <= 1e-15) and np.all(tr["d_dir"] <= 1e-15)


@pytest.mark.parametrize("k", [1, 3, 7])
def test_scale_only_jump(k):
    # V = e1 in blocks 0..k-1, V = 2 e1 in block k: O_k = (k+2)/(k+1) e1
    D = 4
    e1 = np.eye(D, dtype=np.float32)[0]
    case = _blocks_case([e1] * k + [2 * e1], D)
    tr = _traj(case)
    assert tr["d_mag"][k - 1] == pytest.approx(G[f"scale_jump_dmag_k{k}"], rel=1e-15)
    assert tr["d_dir"][k - 1] == 0.0
    # all earlier tests see an unchanged output
    assert np.all(tr["d_mag"][: k - 1] == 0.0)


def test_scale_only_jump_threshold_is_strict():
    D = 4
    e1 = np.eye(D, dtype=np.float32)[0]
    k = 3
    case = _blocks_case([e1] * k + [2 * e1] + [2 * e1], D)
    dm = G["scale_jump_dmag_k3"]  # exactly 0.25
    # eps_mag equal to the statistic: the jump block fails (strict <), counter restarts
    r = oracle.art_reference(*oarr(case), eps_mag=dm, eps_dir=1e-9, patience=3, **okw(case))
    assert r["stop"][0, 0] == 5  # tests at t=1,2 pass, t=3 fails -> never reaches 3 in a row
    r = oracle.art_reference(*oarr(case), eps_mag=dm + 1e-12, eps_dir=1e-9, patience=3, **okw(case))
    assert r["stop"][0, 0] == 4  # t=1,2,3 pass
    # a direction threshold alone cannot be met by a pure scale change -> d_dir = 0 passes any eps_dir > 0
    r = oracle.art_reference(*oarr(case), eps_mag=1e-3, eps_dir=1e-300, patience=3, **okw(case))
    assert r["stop"][0, 0] == 5


def test_rotation_cases():
    D = 2
    e1, e2 = np.eye(D, dtype=np.float32)
    case = _blocks_case([e1, e2], D)
    tr = _traj(case)
    assert tr["d_mag"][0] == pytest.approx(G["rot_half_dmag"], rel=1e-14)
    assert tr["d_dir"][0] == pytest.approx(G["rot_half_ddir"], rel=1e-14)
    # sqrt(3) e2 in block 1: |O_1| = |O_0| = 1, direction moves by 60 degrees
    s3 = np.float32(math.sqrt(3.0))
    case = _blocks_case([e1, s3 * e2], D)
    tr = _traj(case)
    assert abs(tr["d_mag"][0]) < 1e-7  # float32 sqrt(3) makes it not exactly 0
    assert tr["d_dir"][0] == pytest.approx(G["rot_60_ddir"], rel=1e-6)


def test_zero_norm_rules():
    D = 3
    z = np.zeros(D, np.float32)
    e1 = np.eye(D, dtype=np.float32)[0]
    tr = _traj(_blocks_case([z, z], D))
    assert (tr["d_mag"][0], tr["d_dir"][0]) == (0.0, 0.0)
    tr = _traj(_blocks_case([z, e1], D))
    assert math.isinf(tr["d_mag"][0]) and tr["d_dir"][0] == 1.0
    tr = _traj(_blocks_case([e1, -e1], D))
    assert (tr["d_mag"][0], tr["d_dir"][0]) == (1.0, 1.0)
    # all-zero values: every test passes -> stop after patience + 1 blocks
    case = _blocks_case([z] * 6, D)
    r = oracle.art_reference(*oarr(case), eps_mag=1e-3, eps_dir=1e-4, patience=2, **okw(case))
    assert r["stop"][0, 0] == 3 and np.all(r["out"][0, 0] == 0.0)


def test_sink_defers_the_stop():
    # constant V, block 0 visited last: no stop before block 0 is folded
    D, n = 4, 6
    c = np.ones(D, np.float32)
    case = _blocks_case([c] * n, D, order=[5, 4, 3, 2, 1, 0])
    r = oracle.art_reference(*oarr(case), eps_mag=1e-3, eps_dir=1e-4, patience=2, **okw(case))
    assert r["stop"][0, 0] == n
    case = _blocks_case([c] * n, D, order=[5, 4, 0, 3, 2, 1])
    r = oracle.art_reference(*oarr(case), eps_mag=1e-3, eps_dir=1e-4, patience=1, **okw(case))
    assert r["stop"][0, 0] == 3  # tests at t=1,2 pass; block 0 folded at t=2
