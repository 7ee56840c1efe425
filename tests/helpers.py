"""Test-only helpers: build paged inputs in float32 storage from logical K/V."""

import numpy as np


def build_case(q, K, V, block_size, seq_lens=None, order=None, page_seed=0, num_kv_heads=None):
    """Page logical K/V [batch, Hkv, L, D] (float32) into [pages, Hkv, B, D] storage.

    ``order``: None -> block 0 then newest to oldest; a callable(n) -> order
    list; or a list of per-sequence orders.  Pages are a random permutation
    drawn from ``page_seed``.  Rows past seq_len are NaN.
    """
    q = np.asarray(q, dtype=np.float32)
    K = np.asarray(K, dtype=np.float32)
    V = np.asarray(V, dtype=np.float32)
    batch, Hkv, Lmax, D = K.shape
    B = int(block_size)
    if seq_lens is None:
        seq_lens = [Lmax] * batch
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    nblk = [(int(L) + B - 1) // B for L in seq_lens]
    maxb = max(1, max(nblk))
    total = sum(nblk)
    rng = np.random.default_rng(page_seed)
    perm = rng.permutation(total).astype(np.int32)
    table = np.full((batch, maxb), -1, np.int32)
    ordr = np.full((batch, maxb), -1, np.int32)
    kp = np.full((max(total, 1), Hkv, B, D), np.nan, np.float32)
    vp = np.full_like(kp, np.nan)
    off = 0
    for s in range(batch):
        n = nblk[s]
        L = int(seq_lens[s])
        table[s, :n] = perm[off:off + n]
        off += n
        if order is None:
            o = [0] + list(range(n - 1, 0, -1)) if n else []
        elif callable(order):
            o = list(order(n))
        else:
            o = list(order[s])
        ordr[s, :n] = o
        for b in range(n):
            lo, hi = b * B, min(b * B + B, L)
            kp[table[s, b], :, : hi - lo] = K[s, :, lo:hi]
            vp[table[s, b], :, : hi - lo] = V[s, :, lo:hi]
    return {
        "q": q, "k_pages": kp, "v_pages": vp, "k_scale": None, "v_scale": None,
        "block_table": table, "block_order": ordr, "seq_lens": seq_lens,
        "block_size": B, "num_kv_heads": Hkv, "q_dtype": "f32", "kv_dtype": "f32",
    }


def okw(case):
    return dict(block_size=case["block_size"], num_kv_heads=case["num_kv_heads"], q_dtype=case["q_dtype"],
                kv_dtype=case["kv_dtype"], k_scale=case.get("k_scale"), v_scale=case.get("v_scale"))


def oarr(case):
    return (case["q"], case["k_pages"], case["v_pages"], case["block_table"], case["block_order"],
            case["seq_lens"])
