"""Comparison rule between a device result and the oracle (test infrastructure only).

The stop decision compares floating-point statistics against thresholds, so a
device that computes in float32 may legitimately decide differently from the
float64 oracle when a statistic lies within a tiny band of its threshold.  The
rule used here:

* every oracle test (position t >= 1) is classified as a definite pass, a
  definite fail, or ambiguous -- ambiguous when flipping a statistic by at
  most ``band`` (absolute) across its threshold could flip the outcome of the
  two-threshold conjunction;
* a device stop ``s_dev`` is accepted iff some assignment of the ambiguous
  tests makes the patience rule fire exactly at ``s_dev``.  Setting the
  ``patience`` tests that end at ``s_dev`` to pass and every other ambiguous
  test to fail is the only assignment that needs checking: failing a test
  never creates an earlier stop, and the window before ``s_dev`` must pass;
* the output is compared at the accepted stop: against the oracle's output
  when the stops agree, otherwise against the oracle's prefix output at the
  device's stop.

Patience/sink semantics follow the ART explainer, Technical Summary 2.3-2.4.
"""

from __future__ import annotations

from typing import Optional

import numpy as np

from .art_oracle import head_stats_trajectory, prefix_output, stop_rule

PASS, AMBIG, FAIL = 1, 0, -1


def classify_tests(d_mag: np.ndarray, d_dir: np.ndarray, eps_mag: float, eps_dir: float,
                   band: float = 1e-5) -> np.ndarray:
    """Three-valued outcome of each test (index i <-> position t = i + 1)."""
    out = np.empty(len(d_mag), dtype=np.int64)
    for i, (dm, dd) in enumerate(zip(d_mag, d_dir)):
        def cond(x, e):
            if x < e - band:
                return PASS
            if x >= e + band:
                return FAIL
            return AMBIG
        a, b = cond(dm, eps_mag), cond(dd, eps_dir)
        if a == FAIL or b == FAIL:
            out[i] = FAIL
        elif a == PASS and b == PASS:
            out[i] = PASS
        else:
            out[i] = AMBIG
    return out


def feasible_stop(status: np.ndarray, sinks: np.ndarray, patience: int, s_dev: int, n: int) -> bool:
    """True iff some resolution of the ambiguous tests yields stop ``s_dev``."""
    if s_dev < 0 or s_dev > n:
        return False
    passes = [None] + [st == PASS for st in status[: n - 1]]
    if s_dev < n:
        lo = s_dev - patience  # positions s_dev-p .. s_dev-1 must pass
        if lo < 1:
            return False
        for t in range(lo, s_dev):
            if status[t - 1] == FAIL:
                return False
            passes[t] = True
    return stop_rule(passes, list(sinks[:n]), patience) == s_dev


def max_rel_err(o: np.ndarray, r: np.ndarray) -> float:
    """max_d |o - r| / max_d |r| (0 when r == o == 0)."""
    den = float(np.max(np.abs(r))) if r.size else 0.0
    num = float(np.max(np.abs(o - r))) if r.size else 0.0
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return num / den


def compare_with_oracle(dev_out: np.ndarray, dev_stop: np.ndarray, inputs: dict, oracle_res: dict, *,
                        eps_mag: float, eps_dir: float, patience: int, band: float = 1e-5,
                        pairs=None) -> dict:
    """Check device (out, stop) against the oracle on the given (s, h) pairs.

    ``inputs`` holds the raw arrays and metadata passed to the oracle
    (q, k_pages, v_pages, block_table, block_order, seq_lens, block_size,
    num_kv_heads, q_dtype, kv_dtype, k_scale, v_scale).  Returns counts and
    the worst output error; ``bad`` lists unexplained stop mismatches.
    """
    kw = dict(block_size=inputs["block_size"], num_kv_heads=inputs["num_kv_heads"],
              q_dtype=inputs["q_dtype"], kv_dtype=inputs["kv_dtype"],
              k_scale=inputs.get("k_scale"), v_scale=inputs.get("v_scale"),
              visit_lens=inputs.get("visit_lens"))
    arrs = (inputs["q"], inputs["k_pages"], inputs["v_pages"], inputs["block_table"],
            inputs["block_order"], inputs["seq_lens"])
    if pairs is None:
        pairs = sorted(oracle_res["heads"].keys())
    n_equal = n_excused = 0
    bad = []
    worst = 0.0
    worst_at: Optional[tuple] = None
    for s, h in pairs:
        so = int(oracle_res["stop"][s, h])
        sg = int(dev_stop[s, h])
        if so == sg:
            n_equal += 1
            ref = oracle_res["out"][s, h]
        else:
            tr = head_stats_trajectory(*arrs, s=s, h=h, eps_mag=eps_mag, eps_dir=eps_dir,
                                       patience=patience, probe=inputs.get("probe_coords"), **kw)
            st = classify_tests(tr["d_mag"], tr["d_dir"], eps_mag, eps_dir, band)
            if feasible_stop(st, tr["sinks"], patience, sg, tr["n"]):
                n_excused += 1
                ref = prefix_output(*arrs, s=s, h=h, nfold=sg, **kw)
            else:
                bad.append((s, h, so, sg))
                continue
        e = max_rel_err(np.asarray(dev_out[s, h], dtype=np.float64), ref)
        if e > worst or worst_at is None:
            worst, worst_at = e, (s, h)
    return {"equal": n_equal, "excused": n_excused, "bad": bad, "max_rel_err": worst,
            "worst_at": worst_at, "checked": len(pairs)}
