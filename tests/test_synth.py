"""Properties of the seeded input generator (the recipe stated in its docstring)."""

import numpy as np
import torch

import oracle
from kv_cache_run_amd import synth, workloads as W


def test_deterministic():
    a = synth.make_case(W.LLAMA3_8B, batch=1, context=300)
    b = synth.make_case(W.LLAMA3_8B, batch=1, context=300)
    for k in ("q", "k_pages", "v_pages", "block_table", "block_order", "seq_lens"):
        assert np.array_equal(a[k], b[k])


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 37.0
    ours = synth._round_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_paging_order_and_tail():
    c = synth.make_case(W.LLAMA3_8B, batch=3, context=1000)  # 1000 = 62 full blocks + 8 rows
    B = c["block_size"]
    n = (1000 + B - 1) // B
    used = np.sort(c["block_table"][:, :n].ravel())
    assert np.array_equal(used, np.arange(c["num_pages"]))
    for s in range(3):
        assert list(c["block_order"][s, :n]) == [0] + list(range(n - 1, 0, -1))
        last = c["block_table"][s, n - 1]
        tail = c["k_pages"][last, :, 1000 - (n - 1) * B:]
        assert np.all(tail == synth.NAN_BF16)


def test_planted_keys_point_along_the_group_query_sum():
    w = W.LLAMA3_8B
    c = synth.make_case(w, batch=2, context=2048)
    g, B, D = w.group, w.block_size, w.head_dim
    q = oracle.decode_bf16(c["q"])
    for (s, k), (pos, alpha) in c["planted"].items():
        assert len(pos) == round(0.03 * 2048)
        qb = q[s, k * g:(k + 1) * g].sum(0)
        want = 8.0 * alpha[:, None] * qb / np.linalg.norm(qb)
        got = oracle.decode_bf16(c["k_pages"][c["block_table"][s, pos // B], k, pos % B])
        assert np.allclose(got, want, rtol=2 ** -8, atol=1e-6)
        # planted score for head h: 8 alpha (q_h . qbar) / (|qbar| sqrt(D))
        for h in range(k * g, (k + 1) * g):
            sc = got @ q[s, h] / np.sqrt(D)
            ref = 8.0 * alpha * (q[s, h] @ qb) / (np.linalg.norm(qb) * np.sqrt(D))
            assert np.allclose(sc, ref, rtol=2e-2)


def test_span_recipe_and_ragged_lengths():
    c = synth.make_case(W.LONG, batch=1, context=8192)
    for (s, k), (pos, alpha) in c["planted"].items():
        assert len(pos) == 20 * 64 and len(np.unique(pos)) == 20 * 64
    r = synth.make_case(W.RAGGED, batch=6, context=(40, 90))
    assert r["seq_lens"].min() >= 40 and r["seq_lens"].max() <= 90
    fr = [len(p) / r["seq_lens"][s] for (s, k), (p, a) in r["planted"].items()]
    assert min(fr) >= 0.0 and max(fr) <= 0.11


def test_fp8_tiles_use_amax_over_448_scales():
    c = synth.make_case(W.QWEN_FP8, batch=2, context=256)
    codes = c["k_pages"]
    mags = np.abs(oracle.decode_e4m3fn(codes))
    # each tile's largest code is +-448 (the amax maps to the top of the range)
    assert np.all(mags.reshape(codes.shape[0], codes.shape[1], -1).max(-1) == 448.0)
    assert np.all(c["k_scale"] > 0) and c["k_scale"].dtype == np.float32


def test_value_heavy_rows_sit_in_the_oldest_quarter_with_the_gain():
    """The value-heavy recipe scales V at round(f L) positions in [B, L/4) by the gain.  Its positions are drawn
    after the first stream's K/V, so that stream matches the same seed without the recipe except at them."""
    w = W.VALUE_HEAVY
    c = synth.make_case(w, batch=2, context=4096)
    plain = synth.make_case(w.scaled(value_heavy=()), batch=2, context=4096)
    B = w.block_size
    f, gain = w.value_heavy
    for (s, k), vpos in c["planted_value"].items():
        assert len(vpos) == round(f * 4096) and len(np.unique(vpos)) == len(vpos)
        assert vpos.min() >= B and vpos.max() < 4096 // 4
    vpos = c["planted_value"][(0, 0)]
    tab = c["block_table"][0]
    assert np.array_equal(c["k_pages"][tab, 0], plain["k_pages"][tab, 0])
    got = oracle.decode_bf16(c["v_pages"][tab, 0]).reshape(-1, w.head_dim)
    ref = oracle.decode_bf16(plain["v_pages"][tab, 0]).reshape(-1, w.head_dim)
    rest = np.setdiff1d(np.arange(4096), vpos)
    assert np.array_equal(got[rest], ref[rest])
    # bf16(gain * x) == gain * bf16(x) for a power-of-two gain
    assert np.array_equal(got[vpos], gain * ref[vpos])


def test_student_t_draws_have_heavier_tails_than_normal():
    """kv_dist="student_t3": unit variance, kurtosis far above the normal's 3."""
    c = synth.make_case(W.HEAVY_TAIL, batch=1, context=8192)
    v = oracle.decode_bf16(c["v_pages"][c["block_table"][0, :512], 0]).ravel()
    assert abs(v.var() - 1.0) < 0.25
    kurt = np.mean((v - v.mean()) ** 4) / v.var() ** 2
    assert kurt > 6.0


def test_recent_recipe_plants_only_among_the_newest_tokens():
    c = synth.make_case(W.RECENT, batch=2, context=4096)
    for (s, k), (pos, alpha) in c["planted"].items():
        assert len(pos) == round(0.01 * 4096) and len(np.unique(pos)) == len(pos)
        assert pos.min() >= 4096 - int(np.ceil(0.05 * 4096))
