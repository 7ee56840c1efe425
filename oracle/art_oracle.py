"""Plain float64 CPU oracle for ART decode attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this module;
it is used by the tests, by ``__graft_entry__.smoke()`` and by the CPU-baseline
leg of ``bench.py``.  It shares no code, table or helper with the HIP library.

What it computes follows "ART: Attention Run-time Termination for Efficient
Large Language Model Decoding" (gist.science explainer of the paper):

* Technical Summary 2.1 (Core Insight): attention is accumulated block by
  block in a streaming (FlashAttention-style) way, so a partial output exists
  after every KV block.
* 2.2 (Stability-Based Termination Criterion): after each block the partial
  output is compared with the previous one by a magnitude statistic and a
  direction statistic; both must be under their thresholds on the same block.
* 2.3 (Patience Mechanism): the test must hold on ``patience`` consecutive
  blocks before the head stops.
* 2.4 (Integration and Correctness): blocks are visited in a caller-given
  order; online softmax makes the order irrelevant to the exact result;
  block 0 (the attention sink) must be folded before any stop; positional
  encoding and the mask are applied before accumulation.

Readings where the page is silent or loose:

* the monitored vector is the whole normalized partial output
  ``O_t = acc_t / l_t`` (not a few probe coordinates);
* magnitude statistic = |‖O_t‖ - ‖O_{t-1}‖| / ‖O_{t-1}‖;
* direction statistic = max(0, 1 - cos(O_t, O_{t-1}));
* both zero norms -> both statistics 0; only the previous norm zero ->
  (inf, 1); only the current norm zero -> (1, 1);
* strict ``<`` against the thresholds, so a zero threshold never passes;
* a test exists from the second folded block on; a failing test resets the
  counter; the head stops after folding the block that brings the counter to
  ``patience`` provided logical block 0 has been folded; ``stop_block`` is
  the number of folded blocks (``n`` if it never stops);
* q-head h reads kv-head ``h // g`` with ``g = Hq / Hkv``;
* softmax scale 1/sqrt(D); tokens at positions >= seq_len are masked;
* fp8 K/V carry one float32 scale per (page, kv-head) tile: value =
  scale * decode(byte).

Storage formats accepted (raw, as the kernel sees them):
``"f32"`` float32 arrays, ``"bf16"`` uint16 bit patterns, ``"fp8_e4m3fn"``
uint8 codes with float32 per-tile scales.
"""

from __future__ import annotations

import math
from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np

# --------------------------------------------------------------------------
# Storage decoding (exact to float64)
# --------------------------------------------------------------------------


def decode_f32(a: np.ndarray) -> np.ndarray:
    """float32 storage -> float64 (exact widening)."""
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64.

    A bfloat16 value is the upper half of an IEEE-754 binary32 word, so the
    exact value is obtained by placing the 16 bits in the high half of a
    32-bit word and reading it as binary32.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def _e4m3fn_value(code: int) -> float:
    """Value of one OCP FP8 E4M3 ("fn": finite + NaN) code.

    OCP 8-bit floating point specification, E4M3: 1 sign bit, 4 exponent bits
    with bias 7, 3 mantissa bits; exponent field 0 encodes subnormals
    (mantissa/8 * 2^(1-7)); there is no infinity; S.1111.111 is NaN, so the
    largest finite magnitude is S.1111.110 = 1.75 * 2^8 = 448.
    """
    s = -1.0 if (code >> 7) & 1 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * (m / 8.0) * 2.0 ** (1 - 7)
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_E4M3FN_TABLE = np.array([_e4m3fn_value(c) for c in range(256)], dtype=np.float64)


def decode_e4m3fn(codes: np.ndarray) -> np.ndarray:
    """FP8 E4M3FN codes (uint8) -> float64 (exact)."""
    return _E4M3FN_TABLE[np.asarray(codes, dtype=np.uint8)]


def _decoder(dtype: str):
    if dtype == "f32":
        return decode_f32
    if dtype == "bf16":
        return decode_bf16
    if dtype == "fp8_e4m3fn":
        return decode_e4m3fn
    raise ValueError(f"unknown storage dtype {dtype!r}")


# --------------------------------------------------------------------------
# The two statistics and the stop rule (Technical Summary 2.2 and 2.3)
# --------------------------------------------------------------------------


def direction_magnitude(o: np.ndarray, o_prev: np.ndarray) -> Tuple[float, float]:
    """(magnitude statistic, direction statistic) between consecutive outputs.

    Magnitude: relative change of the L2 norm, |‖o‖ - ‖o_prev‖| / ‖o_prev‖.
    Direction: cosine deviation, max(0, 1 - <o, o_prev> / (‖o‖ ‖o_prev‖)).
    Zero norms: both zero -> (0, 0); previous zero -> (inf, 1);
    current zero -> (1, 1).
    """
    a = math.sqrt(float(np.dot(o, o)))
    c = math.sqrt(float(np.dot(o_prev, o_prev)))
    if a == 0.0 and c == 0.0:
        return 0.0, 0.0
    if c == 0.0:
        return math.inf, 1.0
    d_mag = abs(a - c) / c
    if a == 0.0:
        return d_mag, 1.0
    d_dir = max(0.0, 1.0 - float(np.dot(o, o_prev)) / (a * c))
    return d_mag, d_dir


def stop_rule(passes: Sequence[Optional[bool]], sinks: Sequence[bool], patience: int) -> int:
    """Number of folded blocks at which the patience rule fires.

    ``passes[t]`` is the outcome of the two-threshold test after folding
    position t (``None`` at t = 0, where no previous output exists);
    ``sinks[t]`` is True when logical block 0 is at visit position t.
    A pass increments the consecutive-pass counter, a fail resets it to 0;
    the rule fires after position t when the counter has reached
    ``patience`` and block 0 has been folded at some position <= t.
    Returns ``len(passes)`` when it never fires.
    """
    if patience < 1:
        raise ValueError("patience must be >= 1")
    cnt = 0
    sink = False
    for t, (ok, sk) in enumerate(zip(passes, sinks)):
        sink = sink or bool(sk)
        if t >= 1:
            cnt = cnt + 1 if ok else 0
        if cnt >= patience and sink:
            return t + 1
    return len(passes)


# --------------------------------------------------------------------------
# Per-head streaming computation
# --------------------------------------------------------------------------


class _Stream:
    """Decoded K/V blocks of one (sequence, kv-head), fetched on demand."""

    def __init__(self, k_pages, v_pages, k_scale, v_scale, kv_dtype, block_table_row,
                 seq_len, block_size, kvh):
        self.kp, self.vp = k_pages, v_pages
        self.ks, self.vs = k_scale, v_scale
        self.dec = _decoder(kv_dtype)
        self.fp8 = kv_dtype == "fp8_e4m3fn"
        self.table = block_table_row
        self.L = int(seq_len)
        self.B = int(block_size)
        self.kvh = int(kvh)
        self.cache: Dict[int, Tuple[np.ndarray, np.ndarray]] = {}

    def block(self, b: int) -> Tuple[np.ndarray, np.ndarray]:
        """K, V rows (float64) of logical block b, valid tokens only."""
        if b not in self.cache:
            pg = int(self.table[b])
            nt = min(self.B, self.L - b * self.B)
            K = self.dec(self.kp[pg, self.kvh, :nt])
            V = self.dec(self.vp[pg, self.kvh, :nt])
            if self.fp8:
                K = K * float(self.ks[pg, self.kvh])
                V = V * float(self.vs[pg, self.kvh])
            self.cache[b] = (K, V)
        return self.cache[b]


def art_head(qv: np.ndarray, stream: _Stream, order: Sequence[int], eps_mag: float,
             eps_dir: float, patience: int, *, run_to_end: bool = False,
             keep_outputs: Iterable[int] = (), probe=None) -> dict:
    """Stream the blocks of one (sequence, q-head) in visit order.

    Each block is folded into an online-softmax state (running max m, running
    denominator l, running numerator acc), the normalized partial output
    O_t = acc / l is compared with O_{t-1}, and the patience rule decides the
    stop.  With ``run_to_end`` the fold continues past the stop so that the
    statistics of every position are recorded (the stop is still the first
    firing).  ``keep_outputs`` lists fold counts whose O is returned.
    ``probe`` (coordinate indices, None = all): the statistics compare only
    those coordinates of O_t and O_{t-1} (a probe vector, Technical Summary
    2.2); the output returned is still the whole vector.
    """
    pidx = None if probe is None else np.asarray(probe, dtype=np.int64)
    D = qv.shape[0]
    n = len(order)
    scale = 1.0 / math.sqrt(D)
    keep = set(int(x) for x in keep_outputs)
    m = -math.inf
    l = 0.0
    acc = np.zeros(D, dtype=np.float64)
    o_prev = None
    o = np.zeros(D, dtype=np.float64)
    cnt = 0
    sink = False
    stop = n
    fired = False
    d_mag_tr: List[float] = []
    d_dir_tr: List[float] = []
    kept: Dict[int, np.ndarray] = {}
    out_at_stop = np.zeros(D, dtype=np.float64)
    for t in range(n):
        b = int(order[t])
        K, V = stream.block(b)
        s = (K @ qv) * scale
        m_new = max(m, float(s.max()))
        alpha = math.exp(m - m_new)  # exp(-inf) = 0 on the first block
        p = np.exp(s - m_new)
        l = l * alpha + float(p.sum())
        acc = acc * alpha + p @ V
        m = m_new
        o = acc / l
        sink = sink or (b == 0)
        if t >= 1:
            dm, dd = direction_magnitude(o, o_prev) if pidx is None else direction_magnitude(o[pidx], o_prev[pidx])
            d_mag_tr.append(dm)
            d_dir_tr.append(dd)
            ok = (dm < eps_mag) and (dd < eps_dir)
            if not fired:
                cnt = cnt + 1 if ok else 0
        o_prev = o
        if (t + 1) in keep:
            kept[t + 1] = o.copy()
        if not fired and cnt >= patience and sink:
            fired = True
            stop = t + 1
            out_at_stop = o.copy()
            if not run_to_end and not (keep and max(keep) > stop):
                break
    if not fired:
        out_at_stop = o.copy() if n > 0 else np.zeros(D, dtype=np.float64)
    return {
        "out": out_at_stop,
        "stop": stop,
        "d_mag": np.array(d_mag_tr, dtype=np.float64),
        "d_dir": np.array(d_dir_tr, dtype=np.float64),
        "sinks": np.array([int(order[t]) == 0 for t in range(n)], dtype=bool),
        "kept": kept,
        "n": n,
    }


def _validate(eps_mag, eps_dir, patience):
    for name, e in (("eps_mag", eps_mag), ("eps_dir", eps_dir)):
        if not (e >= 0.0):  # rejects NaN and negatives
            raise ValueError(f"{name} must be a number >= 0")
    if int(patience) < 1:
        raise ValueError("patience must be >= 1")


def _nblocks(L: int, B: int) -> int:
    return (int(L) + B - 1) // B


def _check_order(order_row: np.ndarray, n: int) -> np.ndarray:
    o = np.asarray(order_row[:n], dtype=np.int64)
    if n and not np.array_equal(np.sort(o), np.arange(n)):
        raise ValueError("block_order row is not a permutation of range(n)")
    return o


def _visited(order_row: np.ndarray, n: int, visit_lens, s: int) -> np.ndarray:
    """Visit order of sequence s: the whole permutation, or -- a pruned cache -- the first visit_lens[s]
    entries (clamped to [0, n]), which must be distinct blocks of [0, n)."""
    if visit_lens is None:
        return _check_order(order_row, n)
    m = min(max(int(visit_lens[s]), 0), n)
    o = np.asarray(order_row[:m], dtype=np.int64)
    if len(np.unique(o)) != m or (m and (o.min() < 0 or o.max() >= n)):
        raise ValueError("visited block_order entries must be distinct blocks of range(n)")
    return o


def art_reference(q, k_pages, v_pages, block_table, block_order, seq_lens, *, block_size: int,
                  num_kv_heads: int, q_dtype: str, kv_dtype: str, eps_mag: float, eps_dir: float,
                  patience: int, k_scale=None, v_scale=None,
                  pairs: Optional[Iterable[Tuple[int, int]]] = None, visit_lens=None, probe=None) -> dict:
    """ART decode for every (sequence, q-head) or for the listed ``pairs``.

    ``visit_lens`` (a pruned cache): sequence s visits only the first visit_lens[s] entries of its order
    row; the rule runs over those blocks alone and ``stop`` counts them.

    Returns ``{"out": float64 [batch, Hq, D] (NaN where not computed),
    "stop": int64 [batch, Hq] (-1 where not computed), "heads": {(s, h): art_head result}}``.
    """
    _validate(eps_mag, eps_dir, patience)
    Q = _decoder(q_dtype)(q)
    batch, Hq, D = Q.shape
    Hkv = int(num_kv_heads)
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    g = Hq // Hkv
    B = int(block_size)
    want = sorted(set(pairs)) if pairs is not None else [(s, h) for s in range(batch) for h in range(Hq)]
    out = np.full((batch, Hq, D), np.nan)
    stop = np.full((batch, Hq), -1, dtype=np.int64)
    res = {}
    by_stream: Dict[Tuple[int, int], List[int]] = {}
    for s, h in want:
        by_stream.setdefault((s, h // g), []).append(h)
    for (s, kvh), heads in sorted(by_stream.items()):
        L = int(seq_lens[s])
        n = _nblocks(L, B)
        order = _visited(block_order[s], n, visit_lens, s)
        st = _Stream(k_pages, v_pages, k_scale, v_scale, kv_dtype, block_table[s], L, B, kvh)
        for h in heads:
            r = art_head(Q[s, h], st, order, eps_mag, eps_dir, patience, probe=probe)
            out[s, h] = r["out"]
            stop[s, h] = r["stop"]
            res[(s, h)] = r
    return {"out": out, "stop": stop, "heads": res}


def head_stats_trajectory(q, k_pages, v_pages, block_table, block_order, seq_lens, *, s: int, h: int,
                          block_size: int, num_kv_heads: int, q_dtype: str, kv_dtype: str,
                          eps_mag: float, eps_dir: float, patience: int, k_scale=None, v_scale=None,
                          keep_outputs: Iterable[int] = (), visit_lens=None, probe=None) -> dict:
    """Run one head over all its visited blocks, recording the statistics at every position."""
    Q = _decoder(q_dtype)(q)
    Hq = Q.shape[1]
    g = Hq // int(num_kv_heads)
    B = int(block_size)
    L = int(seq_lens[s])
    n = _nblocks(L, B)
    order = _visited(block_order[s], n, visit_lens, s)
    st = _Stream(k_pages, v_pages, k_scale, v_scale, kv_dtype, block_table[s], L, B, h // g)
    return art_head(Q[s, h], st, order, eps_mag, eps_dir, patience, run_to_end=True,
                    keep_outputs=keep_outputs, probe=probe)


def prefix_output(q, k_pages, v_pages, block_table, block_order, seq_lens, *, s: int, h: int, nfold: int,
                  block_size: int, num_kv_heads: int, q_dtype: str, kv_dtype: str, k_scale=None,
                  v_scale=None, visit_lens=None) -> np.ndarray:
    """Attention output of (s, h) over the first ``nfold`` blocks of the visit order.

    Computed from the definition (one softmax over all tokens of those
    blocks), not by streaming; zero vector when ``nfold == 0``.
    """
    Q = _decoder(q_dtype)(q)
    Hq, D = Q.shape[1], Q.shape[2]
    g = Hq // int(num_kv_heads)
    B = int(block_size)
    L = int(seq_lens[s])
    n = _nblocks(L, B)
    order = _visited(block_order[s], n, visit_lens, s)
    if nfold == 0:
        return np.zeros(D)
    st = _Stream(k_pages, v_pages, k_scale, v_scale, kv_dtype, block_table[s], L, B, h // g)
    Ks, Vs = zip(*[st.block(int(order[t])) for t in range(nfold)])
    K = np.concatenate(Ks)
    V = np.concatenate(Vs)
    sc = (K @ Q[s, h]) / math.sqrt(D)
    w = np.exp(sc - sc.max())
    return (w @ V) / w.sum()


def full_attention(q, k_pages, v_pages, block_table, seq_lens, *, block_size: int, num_kv_heads: int,
                   q_dtype: str, kv_dtype: str, k_scale=None, v_scale=None,
                   pairs: Optional[Iterable[Tuple[int, int]]] = None, block_order=None,
                   visit_lens=None) -> np.ndarray:
    """Textbook softmax attention of each decode query over all its valid tokens.

    out[s, h] = sum_j softmax_j(K_j . q / sqrt(D)) V_j over logical positions
    j < seq_len[s], with K, V gathered through the block table.  The result
    the streaming method reaches when it never stops.  With ``visit_lens``
    (and ``block_order``) only the tokens of the visited blocks count.
    """
    Q = _decoder(q_dtype)(q)
    batch, Hq, D = Q.shape
    g = Hq // int(num_kv_heads)
    B = int(block_size)
    out = np.full((batch, Hq, D), np.nan)
    want = sorted(set(pairs)) if pairs is not None else [(s, h) for s in range(batch) for h in range(Hq)]
    cache = {}
    for s, h in want:
        L = int(seq_lens[s])
        n = _nblocks(L, B)
        key = (s, h // g)
        if key not in cache:
            st = _Stream(k_pages, v_pages, k_scale, v_scale, kv_dtype, block_table[s], L, B, h // g)
            blocks = range(n) if visit_lens is None else _visited(block_order[s], n, visit_lens, s)
            if len(blocks):
                Ks, Vs = zip(*[st.block(int(b)) for b in blocks])
                cache = {key: (np.concatenate(Ks), np.concatenate(Vs))}
            else:
                cache = {key: (np.zeros((0, D)), np.zeros((0, D)))}
        K, V = cache[key]
        if K.shape[0] == 0:
            out[s, h] = 0.0
            continue
        sc = (K @ Q[s, h]) / math.sqrt(D)
        w = np.exp(sc - sc.max())
        out[s, h] = (w @ V) / w.sum()
    return out
