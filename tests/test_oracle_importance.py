"""Pins of the oracle's importance-first order (reading R28: block 0, then descending max-over-heads score of
the block's mean key, ties to the newer block).

* equal scores (an all-zero summary) reduce to recency-first: block 0, then newest to oldest;
* a block whose summary alone points along a head's query comes right after block 0;
* the order does not depend on page placement, and scaling every summary by c > 0 keeps it;
* the summary is the mean of the block's valid rows (a NaN-filled tail past seq_len is not read), times
  the fp8 tile scale.
"""

import numpy as np
import pytest

import oracle
from kv_cache_run_amd import synth, workloads as W
from tests.helpers import build_case


def _order(case, summary):
    sc = oracle.block_scores(case["q"], summary, case["block_table"], case["seq_lens"],
                             block_size=case["block_size"], num_kv_heads=case["num_kv_heads"],
                             q_dtype=case["q_dtype"])
    return oracle.importance_order(sc, case["seq_lens"], block_size=case["block_size"])


def _summary(case):
    return oracle.block_key_summary(case["k_pages"], case["block_table"], case["seq_lens"],
                                    block_size=case["block_size"], num_kv_heads=case["num_kv_heads"],
                                    kv_dtype=case["kv_dtype"], k_scale=case.get("k_scale"))


def test_equal_scores_are_recency_first():
    case = synth.make_case(W.TINY, batch=1, context=1000)
    n = (1000 + 15) // 16
    z = np.zeros((case["k_pages"].shape[0], 1, 64))
    o = _order(case, z)
    assert list(o[0, :n]) == [0] + list(range(n - 1, 0, -1))


def test_a_single_aligned_block_comes_right_after_block_zero():
    rng = np.random.default_rng(0)
    D, B, L = 16, 4, 64
    q = rng.standard_normal((1, 2, D))
    K = 0.01 * rng.standard_normal((1, 1, L, D))
    j = 7
    K[0, 0, j * B:(j + 1) * B] = 5.0 * q[0, 1] / np.linalg.norm(q[0, 1])  # aligned with head 1 only
    case = build_case(q, K, np.zeros_like(K), B, num_kv_heads=1)
    o = _order(case, _summary(case))
    assert o[0, 0] == 0 and o[0, 1] == j


def test_order_ignores_page_placement_and_summary_scale():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((2, 4, 16))
    K = rng.standard_normal((2, 2, 70, 16))
    a = build_case(q, K, K, 8, seq_lens=[70, 53], page_seed=1)
    b = build_case(q, K, K, 8, seq_lens=[70, 53], page_seed=2)
    oa, ob = _order(a, _summary(a)), _order(b, _summary(b))
    assert np.array_equal(oa, ob)
    assert np.array_equal(_order(a, 3.0 * _summary(a)), oa)


def test_summary_is_the_mean_of_valid_rows():
    case = synth.make_case(W.LLAMA3_8B, batch=1, context=1000)   # last block: 8 valid rows, NaN tail
    sm = _summary(case)
    B = case["block_size"]
    tab = case["block_table"][0]
    last = tab[(1000 - 1) // B]
    rows = oracle.decode_bf16(case["k_pages"][last, 3, :1000 - 62 * B])
    assert np.all(np.isfinite(sm[last])) and np.allclose(sm[last, 3], rows.mean(0), rtol=1e-12)
    f8 = synth.make_case(W.QWEN_FP8, batch=1, context=64)
    s8 = _summary(f8)
    pg = f8["block_table"][0, 1]
    want = oracle.decode_e4m3fn(f8["k_pages"][pg, 2]).mean(0) * f8["k_scale"][pg, 2]
    assert np.allclose(s8[pg, 2], want, rtol=1e-12)


def test_score_is_max_over_heads_with_contiguous_groups():
    """Hand-worked scores for two kv-heads of two query heads each (reading: max over the query heads,
    kv-head h // g, scale 1/sqrt(D)).  Each alternative reading gives another order:

    * mean or sum over the heads puts block 2 (every head scores 2) before block 1 (one head scores 3);
    * kv-head h % g (interleaved groups) sends head 1 to kv-head 1, where block 3 scores 5 for it.
    """
    D = 2
    q = np.array([[[1.0, 0.0], [0.0, 1.0], [-1.0, 0.0], [0.0, -1.0]]], np.float32)  # [1, Hq=4, D]
    summ = np.zeros((4, 2, D))                                                        # [page, Hkv, D]
    summ[1, 0] = [3.0, 0.0]                      # block 1: head 0 scores 3, the other heads 0
    summ[2, 0] = [2.0, 2.0]                      # block 2: heads 0, 1 score 2 ...
    summ[2, 1] = [-2.0, -2.0]                    # ... and heads 2, 3 score 2
    summ[3, 1] = [0.0, 5.0]                      # block 3: head 2 scores 0, head 3 scores -5
    table = np.array([[0, 1, 2, 3]], np.int32)   # logical block b on page b
    lens = np.array([4], np.int32)
    sc = oracle.block_scores(q, summ, table, lens, block_size=1, num_kv_heads=2, q_dtype="f32")
    r2 = np.sqrt(2.0)
    assert np.allclose(sc[0, 1:], [3.0 / r2, 2.0 / r2, 0.0], rtol=0, atol=1e-15)
    o = oracle.importance_order(sc, lens, block_size=1)
    assert list(o[0]) == [0, 1, 2, 3]
    # the alternatives, written out by hand, would order the blocks otherwise
    mean_scores = {1: 0.75, 2: 2.0, 3: -1.25}
    assert sorted(mean_scores, key=lambda b: -mean_scores[b]) == [2, 1, 3]
    interleaved = {1: 3.0, 2: 2.0, 3: 5.0}       # max over heads with kv-head h % g
    assert sorted(interleaved, key=lambda b: -interleaved[b]) == [3, 1, 2]
