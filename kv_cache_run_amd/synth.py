"""Seeded synthetic inputs for ART decode attention (shared by tests and benchmark).

This module only *makes inputs*: it draws Gaussian q/K/V, plants heavy keys,
rounds to the storage type, pages the cache and writes the visit order.  It
contains none of the method's arithmetic (no scores, softmax, statistics or
stop rule), and neither the oracle nor the HIP library imports it.

Recipe (fixed draw order from ``numpy.random.Generator(PCG64(seed))``):

1. ``seq_lens``: the fixed context, or per sequence an integer drawn
   uniformly from [lo, hi] (inclusive).
2. ``q`` ~ N(0, 1) of shape [batch, Hq, D], rounded to the q storage type.
3. For each stream (sequence s, kv-head k), in that order:
   a. K, V ~ N(0, 1) of shape [L_s, D] (float32 draws), or Student-t with 3
      degrees of freedom divided by sqrt(3) (unit variance, heavy tails) for
      ``kv_dist = "student_t3"``;
   b. the heavy-key positions: ``round(f * L_s)`` distinct positions for
      ("frac", f); for ("frac_range", lo, hi) first f ~ U(lo, hi) per stream;
      for ("spans", c, w) c non-overlapping spans of w tokens with uniformly
      drawn starts (redrawn on overlap); for ("recent", f, w) ``round(f * L_s)``
      distinct positions among the newest ``ceil(w * L_s)`` tokens;
   c. alpha ~ U(2, 4) per heavy position; K at that position becomes
      ``8 * alpha * qbar / |qbar|`` where qbar is the sum of the stored q
      vectors of the kv-head's query group;
   d. only for workloads that ask for them, after c: value-heavy positions,
      ``round(f * L_s)`` distinct positions drawn uniformly from the oldest
      quarter [B, L_s / 4) (block 0 excluded), whose V rows are multiplied by
      ``gain``;
   e. K and V are rounded to the KV storage type (bfloat16: round to nearest
      even; fp8 E4M3FN: per (page, kv-head) tile scale = amax / 448, or 1 for
      an all-zero tile, code = nearest-even E4M3FN of value / scale clamped
      to +-448).
4. Physical pages: one random permutation of [0, total blocks) handed out
   in (sequence, logical block) order.
5. Visit order per sequence: logical block 0 first, then the newest block
   down to block 1.

Rows of the last page past ``seq_len`` are filled with NaN bit patterns so
that any read of a masked row shows up in the output.
"""

from __future__ import annotations

from typing import Optional

import numpy as np

from .workloads import Workload

NAN_BF16 = np.uint16(0x7FC0)
NAN_E4M3FN = np.uint8(0x7F)


def _round_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit pattern, round to nearest even (finite inputs)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    return ((b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def _bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _to_e4m3fn_codes(x: np.ndarray) -> np.ndarray:
    """float32 -> E4M3FN codes via torch's CPU cast (nearest even), after clamping to +-448."""
    import torch

    t = torch.from_numpy(np.clip(np.ascontiguousarray(x, dtype=np.float32), -448.0, 448.0))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _heavy_positions(rng: np.random.Generator, heavy: tuple, L: int) -> np.ndarray:
    kind = heavy[0]
    if kind == "frac":
        cnt = int(round(heavy[1] * L))
        return np.sort(rng.choice(L, size=min(cnt, L), replace=False))
    if kind == "frac_range":
        f = rng.uniform(heavy[1], heavy[2])
        cnt = int(round(f * L))
        return np.sort(rng.choice(L, size=min(cnt, L), replace=False))
    if kind == "recent":
        # round(f * L) distinct positions among the newest ceil(w * L) tokens
        span = min(L, max(1, int(np.ceil(heavy[2] * L))))
        cnt = min(int(round(heavy[1] * L)), span)
        return np.sort(L - span + rng.choice(span, size=cnt, replace=False))
    if kind == "spans":
        count, width = int(heavy[1]), int(heavy[2])
        starts = []
        while len(starts) < count:
            st = int(rng.integers(0, L - width + 1))
            if all(abs(st - o) >= width for o in starts):
                starts.append(st)
        starts.sort()
        return np.concatenate([np.arange(s, s + width) for s in starts])
    raise ValueError(f"unknown heavy-key recipe {heavy!r}")


def make_case(w: Workload, *, seed: Optional[int] = None, batch: Optional[int] = None,
              context=None, tail_fill: Optional[bool] = None) -> dict:
    """Build one decode step of workload ``w`` (optionally with overrides).

    Returns a dict of host NumPy arrays in their storage types plus metadata:
    q [batch, Hq, D]; k_pages/v_pages [num_pages, Hkv, B, D]; k_scale/v_scale
    [num_pages, Hkv] float32 (fp8 only, else None); block_table/block_order
    int32 [batch, max_blocks] (padding -1); seq_lens int32 [batch].
    """
    seed = w.seed if seed is None else seed
    batch = w.batch if batch is None else batch
    context = w.context if context is None else context
    tail_fill = w.tail_fill if tail_fill is None else tail_fill
    rng = np.random.Generator(np.random.PCG64(seed))
    Hq, Hkv, D, B = w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size
    g = Hq // Hkv

    # 1. sequence lengths
    if isinstance(context, tuple):
        seq_lens = rng.integers(context[0], context[1], size=batch, endpoint=True).astype(np.int32)
    else:
        seq_lens = np.full(batch, int(context), dtype=np.int32)
    nblk = (seq_lens.astype(np.int64) + B - 1) // B
    max_blocks = int(max(1, nblk.max()))
    num_pages = int(nblk.sum())

    # 2. queries
    q32 = rng.standard_normal((batch, Hq, D), dtype=np.float32)
    if w.q_dtype == "bf16":
        q = _round_bf16_bits(q32)
        q_vals = _bf16_bits_to_f32(q).astype(np.float64)
    elif w.q_dtype == "f32":
        q = q32
        q_vals = q32.astype(np.float64)
    else:
        raise ValueError(w.q_dtype)

    # 4 (drawn up front so that the page map does not depend on K/V draws)
    perm = rng.permutation(num_pages).astype(np.int32)
    block_table = np.full((batch, max_blocks), -1, dtype=np.int32)
    off = 0
    for s in range(batch):
        block_table[s, : nblk[s]] = perm[off: off + nblk[s]]
        off += int(nblk[s])
    block_order = np.full((batch, max_blocks), -1, dtype=np.int32)
    for s in range(batch):
        n = int(nblk[s])
        if n:
            block_order[s, 0] = 0
            block_order[s, 1:n] = np.arange(n - 1, 0, -1, dtype=np.int32)

    if w.kv_dtype == "bf16":
        kst = np.empty((num_pages, Hkv, B, D), dtype=np.uint16)
        vst = np.empty_like(kst)
        k_scale = v_scale = None
    elif w.kv_dtype == "f32":
        kst = np.empty((num_pages, Hkv, B, D), dtype=np.float32)
        vst = np.empty_like(kst)
        k_scale = v_scale = None
    elif w.kv_dtype == "fp8_e4m3fn":
        kst = np.empty((num_pages, Hkv, B, D), dtype=np.uint8)
        vst = np.empty_like(kst)
        k_scale = np.ones((num_pages, Hkv), dtype=np.float32)
        v_scale = np.ones((num_pages, Hkv), dtype=np.float32)
    else:
        raise ValueError(w.kv_dtype)

    planted = {}
    planted_value = {}
    # 3. per stream K/V, heavy keys, storage rounding, paging
    for s in range(batch):
        L = int(seq_lens[s])
        n = int(nblk[s])
        pages = block_table[s, :n].astype(np.int64)
        for k in range(Hkv):
            if w.kv_dist == "normal":
                K = rng.standard_normal((L, D), dtype=np.float32)
                V = rng.standard_normal((L, D), dtype=np.float32)
            elif w.kv_dist == "student_t3":
                K = (rng.standard_t(3.0, size=(L, D)) / np.sqrt(3.0)).astype(np.float32)
                V = (rng.standard_t(3.0, size=(L, D)) / np.sqrt(3.0)).astype(np.float32)
            else:
                raise ValueError(w.kv_dist)
            pos = _heavy_positions(rng, w.heavy, L)
            alpha = rng.uniform(2.0, 4.0, size=len(pos))
            qbar = q_vals[s, k * g:(k + 1) * g].sum(axis=0)
            nq = float(np.sqrt(qbar @ qbar))
            if len(pos):
                K[pos] = (8.0 * alpha[:, None] * (qbar / nq)[None, :]).astype(np.float32)
            planted[(s, k)] = (pos, alpha)
            if w.value_heavy:
                f, gain = w.value_heavy
                lo, hi = min(B, L), max(min(B, L), L // 4)
                cnt = min(int(round(f * L)), hi - lo)
                vpos = np.sort(rng.choice(np.arange(lo, hi), size=cnt, replace=False)) if cnt > 0 else np.zeros(0, np.int64)
                V[vpos] *= np.float32(gain)
                planted_value[(s, k)] = vpos
            pad = n * B - L
            Kp = np.concatenate([K, np.zeros((pad, D), np.float32)]).reshape(n, B, D)
            Vp = np.concatenate([V, np.zeros((pad, D), np.float32)]).reshape(n, B, D)
            if w.kv_dtype == "bf16":
                kb, vb = _round_bf16_bits(Kp), _round_bf16_bits(Vp)
                if pad and tail_fill:
                    kb[n - 1, B - pad:] = NAN_BF16
                    vb[n - 1, B - pad:] = NAN_BF16
            elif w.kv_dtype == "f32":
                kb, vb = Kp.copy(), Vp.copy()
                if pad and tail_fill:
                    kb[n - 1, B - pad:] = np.nan
                    vb[n - 1, B - pad:] = np.nan
            else:
                ka = np.abs(Kp).reshape(n, -1).max(axis=1)
                va = np.abs(Vp).reshape(n, -1).max(axis=1)
                ks = np.where(ka > 0, ka / 448.0, 1.0).astype(np.float32)
                vs = np.where(va > 0, va / 448.0, 1.0).astype(np.float32)
                kb = _to_e4m3fn_codes(Kp / ks[:, None, None])
                vb = _to_e4m3fn_codes(Vp / vs[:, None, None])
                if pad and tail_fill:
                    kb[n - 1, B - pad:] = NAN_E4M3FN
                    vb[n - 1, B - pad:] = NAN_E4M3FN
                k_scale[pages, k] = ks
                v_scale[pages, k] = vs
            kst[pages, k] = kb
            vst[pages, k] = vb

    return {
        "workload": w.name,
        "q": q, "k_pages": kst, "v_pages": vst, "k_scale": k_scale, "v_scale": v_scale,
        "block_table": block_table, "block_order": block_order, "seq_lens": seq_lens,
        "batch": batch, "num_q_heads": Hq, "num_kv_heads": Hkv, "head_dim": D, "block_size": B,
        "q_dtype": w.q_dtype, "kv_dtype": w.kv_dtype, "max_blocks": max_blocks, "num_pages": num_pages,
        "eps_mag": w.eps_mag, "eps_dir": w.eps_dir, "patience": w.patience,
        "planted": planted, "planted_value": planted_value,
    }


def oracle_kwargs(case: dict) -> dict:
    """Keyword arguments shared by the oracle entry points (``visit_lens`` when the case prunes its cache)."""
    kw = dict(block_size=case["block_size"], num_kv_heads=case["num_kv_heads"], q_dtype=case["q_dtype"],
              kv_dtype=case["kv_dtype"], k_scale=case["k_scale"], v_scale=case["v_scale"])
    if case.get("visit_lens") is not None:
        kw["visit_lens"] = case["visit_lens"]
    return kw


def oracle_detector_kwargs(case: dict) -> dict:
    """The probe coordinates for the oracle's detector when the case asks for a probe vector."""
    return {} if case.get("probe_coords") is None else {"probe": case["probe_coords"]}


def oracle_arrays(case: dict) -> tuple:
    return (case["q"], case["k_pages"], case["v_pages"], case["block_table"], case["block_order"],
            case["seq_lens"])
