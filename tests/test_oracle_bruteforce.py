"""Pin the streaming oracle to definitions it does not share code with.

* every partial output O_t equals softmax attention recomputed from scratch
  over the tokens of the blocks visited so far (brute force);
* the never-stopping result equals torch's float64 scaled_dot_product_attention
  (a library routine) with grouped KV heads expanded by ``repeat_interleave``.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from tests.helpers import build_case, oarr, okw


def _rand_case(seed, batch=2, Hq=4, Hkv=2, D=16, B=4, lens=(37, 24), order="default"):
    rng = np.random.default_rng(seed)
    Lmax = max(lens)
    q = rng.standard_normal((batch, Hq, D)).astype(np.float32)
    K = (2.0 * rng.standard_normal((batch, Hkv, Lmax, D))).astype(np.float32)
    V = rng.standard_normal((batch, Hkv, Lmax, D)).astype(np.float32)
    if order == "default":
        od = None
    elif order == "identity":
        od = lambda n: range(n)  # noqa: E731
    else:
        od = [list(rng.permutation((L + B - 1) // B)) for L in lens]
    return build_case(q, K, V, B, seq_lens=lens, order=od, page_seed=seed), (q, K, V)


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("order", ["default", "identity", "random"])
def test_every_partial_output_matches_bruteforce(seed, order):
    case, (q, K, V) = _rand_case(seed, order=order)
    B = case["block_size"]
    g = q.shape[1] // K.shape[1]
    for s in range(q.shape[0]):
        L = int(case["seq_lens"][s])
        n = (L + B - 1) // B
        ordr = case["block_order"][s, :n]
        for h in range(q.shape[1]):
            tr = oracle.head_stats_trajectory(*oarr(case), s=s, h=h, eps_mag=1e-3, eps_dir=1e-4, patience=2,
                                              keep_outputs=range(1, n + 1), **okw(case))
            bf = oracle.prefix_attention_bruteforce(q[s, h].astype(np.float64), K[s, h // g, :L].astype(np.float64),
                                                    V[s, h // g, :L].astype(np.float64), ordr, B, L)
            for t in range(n):
                got = tr["kept"][t + 1]
                assert np.allclose(got, bf[t], rtol=1e-12, atol=1e-13), (s, h, t)
                # statistics recorded at t are functions of O_t and O_{t-1} of the definition
                if t >= 1:
                    dm, dd = oracle.direction_magnitude(bf[t], bf[t - 1])
                    assert abs(dm - tr["d_mag"][t - 1]) <= 1e-12 * max(1.0, dm)
                    assert abs(dd - tr["d_dir"][t - 1]) <= 1e-12


@pytest.mark.parametrize("seed", [3, 4])
def test_full_attention_matches_torch_sdpa_float64(seed):
    case, (q, K, V) = _rand_case(seed, batch=3, Hq=6, Hkv=2, D=8, B=4, lens=(13, 32, 1))
    ref = np.zeros(q.shape)
    g = 3
    for s in range(3):
        L = int(case["seq_lens"][s])
        qt = torch.from_numpy(q[s].astype(np.float64))[:, None, :]  # [Hq, 1, D]
        kt = torch.from_numpy(K[s, :, :L].astype(np.float64)).repeat_interleave(g, dim=0)
        vt = torch.from_numpy(V[s, :, :L].astype(np.float64)).repeat_interleave(g, dim=0)
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=1.0 / math.sqrt(8))
        ref[s] = o[:, 0, :].numpy()
    full = oracle.full_attention(case["q"], case["k_pages"], case["v_pages"], case["block_table"],
                                 case["seq_lens"], **okw(case))
    assert np.allclose(full, ref, rtol=1e-12, atol=1e-14)
    # the streaming rule with a zero threshold never stops and reaches the same result
    r = oracle.art_reference(*oarr(case), eps_mag=0.0, eps_dir=1e-4, patience=1, **okw(case))
    assert np.allclose(r["out"], ref, rtol=1e-12, atol=1e-14)
    n = (case["seq_lens"] + 3) // 4
    assert np.array_equal(r["stop"], np.repeat(n[:, None], 6, axis=1))


def test_prefix_output_matches_streaming():
    case, _ = _rand_case(5, order="random")
    for nfold in (1, 3, 7):
        tr = oracle.head_stats_trajectory(*oarr(case), s=0, h=1, eps_mag=1e-3, eps_dir=1e-4, patience=2,
                                          keep_outputs=[nfold], **okw(case))
        p = oracle.prefix_output(*oarr(case), s=0, h=1, nfold=nfold, **okw(case))
        assert np.allclose(tr["kept"][nfold], p, rtol=1e-12, atol=1e-14)


def test_zero_length_sequence_gives_zero_output_and_zero_stop():
    case, _ = _rand_case(6, lens=(0, 9))
    r = oracle.art_reference(*oarr(case), eps_mag=1e-3, eps_dir=1e-4, patience=1, **okw(case))
    assert np.all(r["stop"][0] == 0) and np.all(r["out"][0] == 0.0)
    assert np.all(np.isfinite(r["out"][1]))
