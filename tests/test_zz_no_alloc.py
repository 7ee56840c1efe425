"""The no-allocation entry point (art_decode_noalloc): its outputs against art_decode's on the same inputs,
through the C ABI, on two calls in a row with the second smaller (the static scratch keeps the first call's
contents).  Full attention uses the scratch for its split partials; ART mode runs the stream kernel (groups of
up to 8 heads) or the scanners without helpers (larger groups), which art_decode runs with the same knobs."""

import numpy as np
import pytest

import oracle
from kv_cache_run_amd import synth, workloads as W

pytestmark = pytest.mark.gpu


def _run(case, em, ed, p, noalloc, env=None):
    import os

    import torch

    from kv_cache_run_amd import art

    old = {k: os.environ.get(k) for k in (env or {})}
    os.environ.update(env or {})
    art.reload_environment()
    try:
        dev = art.case_to_device(case)
        out = torch.full((case["batch"], case["num_q_heads"], case["head_dim"]), float("nan"), device="cuda")
        stop = torch.full((case["batch"], case["num_q_heads"]), -7, dtype=torch.int32, device="cuda")
        fetched = torch.full((case["batch"], case["num_kv_heads"]), -7, dtype=torch.int32, device="cuda")
        args = (dev["q"], dev["k_pages"], dev["v_pages"], dev["block_table"], dev["block_order"], dev["seq_lens"],
                em, ed, p, out, stop)
        if noalloc:
            art.art_decode_noalloc(*args, k_scale=dev["k_scale"], v_scale=dev["v_scale"], blocks_fetched=fetched)
        else:
            dec = art.Decoder(dev["q"], dev["k_pages"], dev["block_table"])
            dec(*args[:9], k_scale=dev["k_scale"], v_scale=dev["v_scale"], out=out, stop_block=stop,
                blocks_fetched=fetched)
        torch.cuda.synchronize()
        return out.cpu().numpy(), stop.cpu().numpy(), fetched.cpu().numpy()
    finally:
        for k, v in old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
        art.reload_environment()


CASES = [(W.LLAMA3_8B, dict(batch=4, context=8192 - 5), dict(batch=2, context=3000)),
         (W.QWEN_FP8, dict(batch=4, context=16384 - 3), dict(batch=1, context=2000 + 7)),
         (W.LLAMA3_8B.scaled(name="bf16-gqa16", num_q_heads=128), dict(batch=2, context=4000),
          dict(batch=1, context=1000))]


@pytest.mark.parametrize("w,big,small", CASES, ids=["bf16-gqa4", "fp8-gqa7", "bf16-gqa16"])
def test_noalloc_matches_art_decode_on_two_calls(w, big, small):
    g = w.num_q_heads // w.num_kv_heads
    env = dict(ART_SCHED="stream") if g <= 8 else dict(ART_SCHED="scan", ART_HELPERS="0")
    for kw in (big, small):
        case = synth.make_case(w, **kw)
        em, ed, p = case["eps_mag"], case["eps_dir"], case["patience"]
        print(f"[noalloc] {case['workload']} batch={case['batch']}", flush=True)
        # full attention: the split partials go through the static scratch
        a = _run(case, 0.0, 0.0, 1, True)
        b = _run(case, 0.0, 0.0, 1, False)
        assert all(np.array_equal(x, y) for x, y in zip(a, b))
        ref = oracle.full_attention(case["q"], case["k_pages"], case["v_pages"], case["block_table"],
                                    case["seq_lens"], **synth.oracle_kwargs(case))
        assert max(oracle.feasible.max_rel_err(a[0][s, h], ref[s, h]) for s in range(case["batch"])
                   for h in range(case["num_q_heads"])) <= 2e-3
        # ART mode: the same kernel art_decode runs with those knobs
        a = _run(case, em, ed, p, True)
        b = _run(case, em, ed, p, False, env)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
        # blocks read ahead of a stop depend on timing; every block a head of the group folded was read
        n = (case["seq_lens"].astype(np.int64) + case["block_size"] - 1) // case["block_size"]
        grp = a[1].reshape(case["batch"], case["num_kv_heads"], g).max(axis=2)
        assert np.all(a[2] >= grp) and np.all(a[2] <= n[:, None])
        r = oracle.art_reference(*synth.oracle_arrays(case), eps_mag=em, eps_dir=ed, patience=p,
                                 **synth.oracle_kwargs(case))
        rep = oracle.compare_with_oracle(a[0], a[1], case, r, eps_mag=em, eps_dir=ed, patience=p)
        assert rep["bad"] == [] and rep["max_rel_err"] <= 2e-3, rep
