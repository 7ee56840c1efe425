"""Parity of the HIP path (through the C ABI) with the CPU oracle, on one MI355X.

Bars: stop_block bit-exact except where the oracle's statistic lies within
1e-5 of its threshold (feasible-stop rule, oracle/feasible.py); outputs within
2e-3 max relative error at the compared stop; full-attention mode within the
same tolerance.  Every head is compared, at reduced sizes and at the full
benchmark sizes, plus properties that hold at any size.
"""

import math
import zlib

import numpy as np
import pytest

import oracle
from kv_cache_run_amd import synth, workloads as W

pytestmark = pytest.mark.gpu

TOL = 2e-3


def _device_run(case, eps_mag, eps_dir, patience, flags=0, reps=1):
    import torch

    from kv_cache_run_amd import art

    dev = art.case_to_device(case)
    dec = art.Decoder(dev["q"], dev["k_pages"], dev["block_table"])
    fetched = torch.full((case["batch"], case["num_kv_heads"]), -7, dtype=torch.int32, device="cuda")
    vl = None if case.get("visit_lens") is None else torch.from_numpy(case["visit_lens"].astype(np.int32)).cuda()
    if case.get("probe"):
        flags |= art.art_flag_probe(case["probe"])
    outs = []
    for _ in range(reps):
        out, stop = dec(dev["q"], dev["k_pages"], dev["v_pages"], dev["block_table"], dev["block_order"],
                        dev["seq_lens"], eps_mag, eps_dir, patience, k_scale=dev["k_scale"], v_scale=dev["v_scale"],
                        blocks_fetched=fetched, flags=flags, visit_lens=vl)
        torch.cuda.synchronize()
        outs.append((out.cpu().numpy().astype(np.float64), stop.cpu().numpy(), fetched.cpu().numpy()))
    return outs if reps > 1 else outs[0]


def _pairs(case, sample=None, seed=0):
    allp = [(s, h) for s in range(case["batch"]) for h in range(case["num_q_heads"])]
    if sample is None or sample >= len(allp):
        return allp
    rng = np.random.default_rng(seed)
    idx = rng.choice(len(allp), size=sample, replace=False)
    return sorted(allp[i] for i in idx)


def _nblocks(case):
    """Visit positions per sequence: n_s, or the case's visit counts (a pruned cache) clamped to n_s."""
    n = (case["seq_lens"].astype(np.int64) + case["block_size"] - 1) // case["block_size"]
    if case.get("visit_lens") is not None:
        n = np.clip(case["visit_lens"].astype(np.int64), 0, n)
    return n


def check_art(case, eps_mag=None, eps_dir=None, patience=None, sample=None, flags=0):
    em = case["eps_mag"] if eps_mag is None else eps_mag
    ed = case["eps_dir"] if eps_dir is None else eps_dir
    p = case["patience"] if patience is None else patience
    print(f"[art] {case['workload']} batch={case['batch']} eps=({em},{ed}) p={p}", flush=True)
    out, stop, fetched = _device_run(case, em, ed, p, flags=flags)
    pairs = _pairs(case, sample)
    ref = oracle.art_reference(*synth.oracle_arrays(case), eps_mag=em, eps_dir=ed, patience=p,
                               pairs=pairs, **synth.oracle_kwargs(case), **synth.oracle_detector_kwargs(case))
    rep = oracle.compare_with_oracle(out, stop, case, ref, eps_mag=em, eps_dir=ed, patience=p, pairs=pairs)
    assert rep["bad"] == [], rep
    assert rep["max_rel_err"] <= TOL, rep
    # properties at any size: the stream reads at least every block a head of its group folded
    n = _nblocks(case)
    g = case["num_q_heads"] // case["num_kv_heads"]
    grp_max = stop.reshape(case["batch"], case["num_kv_heads"], g).max(axis=2)
    assert np.all(stop >= 0) and np.all(stop <= n[:, None])
    assert np.all(fetched >= grp_max) and np.all(fetched <= n[:, None])
    assert np.all(np.isfinite(out))
    return rep, out, stop, fetched


def check_full(case, sample=None, flags=0):
    print(f"[full] {case['workload']} batch={case['batch']}", flush=True)
    out, stop, fetched = _device_run(case, 0.0, 0.0, 1, flags=flags)
    pairs = _pairs(case, sample)
    ref = oracle.full_attention(case["q"], case["k_pages"], case["v_pages"], case["block_table"], case["seq_lens"],
                                pairs=pairs, block_order=case["block_order"], **synth.oracle_kwargs(case))
    worst = 0.0
    for s, h in pairs:
        worst = max(worst, oracle.feasible.max_rel_err(out[s, h], ref[s, h]))
    n = _nblocks(case)
    assert worst <= TOL, worst
    assert np.array_equal(stop, np.repeat(n[:, None], case["num_q_heads"], axis=1))
    assert np.array_equal(fetched, np.repeat(n[:, None], case["num_kv_heads"], axis=1))
    return worst


# ---- every head, at sizes the oracle finishes in seconds (ragged tails included) -------------------------

REDUCED = [
    (W.TINY, dict()),
    (W.TINY, dict(context=1000)),
    (W.LLAMA3_8B, dict(batch=2, context=8192 - 5)),
    (W.RAGGED, dict(batch=4)),
    (W.LONG, dict(batch=1, context=131072 - 7)),
    (W.QWEN_FP8, dict(batch=4, context=16384 - 3)),
]


@pytest.mark.parametrize("w,kw", REDUCED, ids=[f"{w.name}-{kw}" for w, kw in REDUCED])
def test_art_parity_reduced(w, kw):
    check_art(synth.make_case(w, **kw))


@pytest.mark.parametrize("w,kw", REDUCED, ids=[f"{w.name}-{kw}" for w, kw in REDUCED])
def test_full_parity_reduced(w, kw):
    check_full(synth.make_case(w, **kw))


# ---- shape matrix corners ------------------------------------------------------------------------------

SHAPES = [
    W.LLAMA3_8B.scaled(name="bf16-d64-gqa4", head_dim=64),
    W.LLAMA3_8B.scaled(name="bf16-blk32-gqa4", block_size=32),
    W.LLAMA3_8B.scaled(name="bf16-mha", num_q_heads=8),
    W.LLAMA3_8B.scaled(name="bf16-gqa16", num_q_heads=128),
    W.LLAMA3_8B.scaled(name="bf16-gqa2-d64-blk32", num_q_heads=16, head_dim=64, block_size=32),
    W.QWEN_FP8.scaled(name="fp8-d64-gqa7", head_dim=64),
    W.QWEN_FP8.scaled(name="fp8-blk32-gqa7", block_size=32),
    W.TINY.scaled(name="f32-d128-gqa3", head_dim=128, num_q_heads=6, num_kv_heads=2),
    W.TINY.scaled(name="f32-d64-blk32-gqa12", num_q_heads=12, block_size=32),
]


@pytest.mark.parametrize("w", SHAPES, ids=[w.name for w in SHAPES])
def test_shape_matrix(w):
    case = synth.make_case(w, batch=2, context=2000 + 9)
    check_art(case)
    check_full(case)


# ---- edge cases ----------------------------------------------------------------------------------------


def _with_lens(case, lens):
    """Shorten sequences; each order row becomes block 0 then newest to oldest of the new length."""
    c = dict(case)
    c["seq_lens"] = np.asarray(lens, dtype=np.int32)
    order = np.full_like(case["block_order"], -1)
    for s, L in enumerate(lens):
        n = (int(L) + case["block_size"] - 1) // case["block_size"]
        if n:
            order[s, :n] = [0] + list(range(n - 1, 0, -1))
    c["block_order"] = order
    return c


def test_empty_short_and_single_token_sequences():
    base = synth.make_case(W.LLAMA3_8B, batch=5, context=700)
    case = _with_lens(base, [0, 1, 15, 16, 17])
    check_art(case, patience=1, eps_mag=0.5, eps_dir=0.5)
    check_art(case)
    check_full(case)
    out, stop, fetched = _device_run(case, 1e-3, 1e-4, 4)
    assert np.all(out[0] == 0.0) and np.all(stop[0] == 0) and np.all(fetched[0] == 0)


@pytest.mark.parametrize("wgs", ["1", "3", "7", "256", "1000", "5000"])
def test_full_attention_over_any_workgroup_count(wgs):
    """Full attention partitions the flattened block list over ART_FULL_WGS workgroups: one workgroup
    folding every stream, counts that cut streams at odd places, more workgroups than blocks (some get none)
    and many pieces per stream all match the oracle on every head, with empty and one-block sequences mixed
    into a ragged batch."""
    base = synth.make_case(W.RAGGED, batch=6)
    lens = [int(x) for x in base["seq_lens"]]
    lens[1] = 0
    lens[3] = 1
    case = _with_lens(base, lens)
    _with_env(dict(ART_FULL_WGS=wgs), lambda: check_full(case))
    out, stop, fetched = _with_env(dict(ART_FULL_WGS=wgs), lambda: _device_run(case, 0.0, 0.0, 1))
    assert np.all(out[1] == 0.0) and np.all(stop[1] == 0) and np.all(fetched[1] == 0)


def test_sink_not_first_and_random_orders():
    case = synth.make_case(W.LLAMA3_8B, batch=3, context=3000)
    rng = np.random.default_rng(11)
    n = int(_nblocks(case)[0])
    order = case["block_order"].copy()
    order[0, :n] = list(range(n - 1, -1, -1))  # block 0 last: nobody can stop early
    order[1, :n] = rng.permutation(n)
    order[2, :n] = [5, 4, 3, 2, 1, 0] + list(range(6, n))
    case["block_order"] = order
    rep, out, stop, fetched = check_art(case, eps_mag=1e-2, eps_dir=1e-3, patience=2)
    assert np.all(stop[0] == n)


def test_patience_one_and_loose_thresholds():
    case = synth.make_case(W.LLAMA3_8B, batch=2, context=4096)
    rep, out, stop, fetched = check_art(case, eps_mag=10.0, eps_dir=10.0, patience=1)
    assert np.all(stop == 2)  # every test passes: stop right after the first test
    check_art(case, eps_mag=10.0, eps_dir=10.0, patience=5)


def test_zero_threshold_keeps_detector_and_equals_full():
    from kv_cache_run_amd import art

    case = synth.make_case(W.LLAMA3_8B, batch=1, context=1024 + 3)
    rep, out, stop, fetched = check_art(case, eps_mag=0.0, eps_dir=1e-4, flags=art.ART_FLAG_KEEP_DETECTOR)
    assert np.all(stop == _nblocks(case)[0])
    check_full(case, flags=art.ART_FLAG_FULL)


def test_stop_monotone_in_thresholds_on_device():
    case = synth.make_case(W.LLAMA3_8B, batch=2, context=8192)
    prev = None
    for em, ed in [(1e-4, 1e-5), (5e-4, 5e-5), (1e-3, 1e-4), (4e-3, 4e-4), (1.6e-2, 1.6e-3)]:
        _, stop, _ = _device_run(case, em, ed, 4)
        if prev is not None:
            assert np.all(stop <= prev)
        prev = stop


def test_repeatable_and_workspace_reusable():
    case = synth.make_case(W.RAGGED, batch=3)
    runs = _device_run(case, 0.0, 0.0, 1, reps=3)
    for o, s, f in runs[1:]:
        assert np.array_equal(o, runs[0][0]) and np.array_equal(s, runs[0][1])
    runs = _device_run(case, 1e-3, 1e-4, 4, reps=2)
    assert np.array_equal(runs[0][0], runs[1][0]) and np.array_equal(runs[0][1], runs[1][1])


# ---- full sizes (the benchmark shapes): every head ------------------------------------------------------

FULL_SIZES = [W.LLAMA3_8B, W.RAGGED, W.LONG, W.QWEN_FP8]


@pytest.mark.parametrize("w", FULL_SIZES, ids=[w.name for w in FULL_SIZES])
def test_full_size_every_head(w):
    """The benchmark shapes at full size, in the launch configuration bench.py times: every head's stop and
    output against the oracle (ART mode stops early, so the float64 oracle finishes in seconds), and every
    head's full-attention output."""
    case = synth.make_case(w)
    rep, _, _, _ = check_art(case)
    assert rep["checked"] == case["batch"] * case["num_q_heads"]
    check_full(case)


# ---- the workgroup schedulers ---------------------------------------------------------------------------
#
# Look-back scheduler: the state entering a chunk is the left fold of the chunk aggregates before it,
# whichever published inclusive state the look-back starts from, so the results are bit-identical whatever the
# number of workers, the window or the timing.  Scanners: partials are computed by the same code
# whichever workgroup (scanner or helper) takes a chunk and the scanner folds them in visit order, so results
# are bit-identical across helper configurations.

LB_VARIANTS = [
    dict(ART_SCHED="lb"),                                     # defaults
    dict(ART_SCHED="lb", ART_WORKERS="1"),                    # one worker: every item in claim order
    dict(ART_SCHED="lb", ART_WINDOW="1"),                     # one chunk past the resolved frontier
    dict(ART_SCHED="lb", ART_WINDOW="2", ART_WORKERS="3"),
    dict(ART_SCHED="lb", ART_WINDOW="32", ART_WORKERS="5000"),  # more workgroups than resident slots
]
SCAN_VARIANTS = [
    dict(ART_SCHED="scan", ART_HELPERS="0"),                  # scanners only
    dict(ART_SCHED="scan", ART_HELPERS="-1"),                 # default helper count
    dict(ART_SCHED="scan", ART_HELPERS="2000", ART_RING="2", ART_LOOKAHEAD="2"),  # many helpers, tight ring
    dict(ART_SCHED="scan", ART_HELPERS="64", ART_RING="1", ART_LOOKAHEAD="1"),    # one slot per stream
    dict(ART_SCHED="scan", ART_HELPERS="300", ART_RING="16", ART_LOOKAHEAD="16"),  # deep speculation
]


STREAM_VARIANTS = [
    dict(ART_SCHED="stream"),                                 # defaults: lookahead 32 + frontier / 2
    dict(ART_SCHED="stream", ART_LA0="1", ART_LA_SHIFT="30"),   # the smallest lookahead (two chunks)
    dict(ART_SCHED="stream", ART_LA0="100000", ART_LA_SHIFT="0"),  # the largest (ring and register ring)
    dict(ART_SCHED="stream", ART_LA0="24", ART_LA_SHIFT="3"),
]


SEG_VARIANTS = [
    dict(ART_SCHED="seg"),                                    # defaults: two segments past the frontier + half of it
    dict(ART_SCHED="seg", ART_SEG_WIN="1"),                   # the smallest window
    dict(ART_SCHED="seg", ART_SEG_WIN="64"),                  # every segment at once
    dict(ART_SCHED="seg", ART_SEG_WGS="7"),                   # few workgroups: long queues of items each
    dict(ART_SCHED="seg", ART_SEG_WGS="1000"),                # more workgroups than CUs
    dict(ART_SCHED="seg", ART_SEG_EXT="0"),                   # no claims past the window
    dict(ART_SCHED="seg", ART_SEG_EXT="4096", ART_SEG_WIN="1"),   # idle claims without bound
    dict(ART_SCHED="seg", ART_SEG_EXT="4096", ART_SEG_WGS="7"),   # few workgroups, unbounded idle claims
]


WIN_VARIANTS = [
    dict(ART_SCHED="win"),                                    # default: two fold workgroups when heads are few
    dict(ART_SCHED="win", ART_WIN_SPLIT="1"),                 # one fold workgroup per (stream, head)
    dict(ART_SCHED="win", ART_WIN_SPLIT="2"),
    dict(ART_SCHED="win", ART_WIN_SPLIT="4"),                 # a 64-chunk window over four workgroups
    dict(ART_SCHED="win", ART_WIN_FIRST="2", ART_WIN_GROWTH="2"),   # windows 2, 4, 8, ...
    dict(ART_SCHED="win", ART_WIN_FIRST="64", ART_WIN_SPLIT="3"),   # every window 64 chunks
    dict(ART_SCHED="win", ART_WIN_FIRST="3", ART_WIN_GROWTH="5"),   # windows 3, 15, 64, ...
]


def _with_env(env, fn):
    """Run fn with the tuning variables in env set (the library re-reads them on each change)."""
    import os

    from kv_cache_run_amd import art

    old = {k: os.environ.get(k) for k in env}
    os.environ.update(env)
    art.reload_environment()
    try:
        return fn()
    finally:
        for k, v in old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
        art.reload_environment()


SCHED_CASES = [(W.LLAMA3_8B, dict(batch=3, context=8192 - 40)), (W.RAGGED, dict(batch=3)),
               (W.QWEN_FP8, dict(batch=2, context=16384 - 3)), (W.LONG, dict(batch=1, context=131072 - 17))]


@pytest.mark.parametrize("variants", [LB_VARIANTS, SCAN_VARIANTS, WIN_VARIANTS, STREAM_VARIANTS, SEG_VARIANTS],
                         ids=["lookback", "scanners", "windowed", "stream", "segments"])
@pytest.mark.parametrize("w,kw", SCHED_CASES, ids=["llama", "ragged", "fp8", "long"])
def test_scheduler_variants_bit_identical(w, kw, variants):
    case = synth.make_case(w, **kw)
    em, ed, p = case["eps_mag"], case["eps_dir"], case["patience"]
    ref = None
    for env in variants:
        print(f"[sched] {case['workload']} {env}", flush=True)
        out, stop, fetched = _with_env(env, lambda: _device_run(case, em, ed, p))
        if ref is None:
            rep, ref_out, ref_stop, _ = _with_env(env, lambda: check_art(case))
            assert np.array_equal(ref_out, out) and np.array_equal(ref_stop, stop)
            ref = (out, stop)
        else:
            assert np.array_equal(out, ref[0]), env
            assert np.array_equal(stop, ref[1]), env
        n = _nblocks(case)
        g = case["num_q_heads"] // case["num_kv_heads"]
        grp_max = stop.reshape(case["batch"], case["num_kv_heads"], g).max(axis=2)
        assert np.all(fetched >= grp_max) and np.all(fetched <= n[:, None]), env


@pytest.mark.parametrize("w,kw", SCHED_CASES, ids=["llama", "ragged", "fp8", "long"])
def test_windowed_and_lookback_give_the_same_bits(w, kw):
    """Both fold the same chunk aggregates left to right and evaluate every position from the state entering
    its chunk with the same arithmetic, so outputs and stops agree bit for bit."""
    case = synth.make_case(w, **kw)
    em, ed, p = case["eps_mag"], case["eps_dir"], case["patience"]
    print(f"[win=lb] {case['workload']}", flush=True)
    a = _with_env(dict(ART_SCHED="lb"), lambda: _device_run(case, em, ed, p))
    b = _with_env(dict(ART_SCHED="win"), lambda: _device_run(case, em, ed, p))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_scheduler_epoch_advances_and_no_error():
    """The look-back scheduler and scanners with helpers advance the stored epoch by one per call and leave
    the finished-workgroup counter at 0 and the error flag clear; scanners without helpers do not touch the
    scheduler words.  Repeated calls give identical results."""
    import torch

    from kv_cache_run_amd import art

    case = synth.make_case(W.RAGGED, batch=2)
    dev = art.case_to_device(case)

    def run(env, expect_epoch):
        dec = _with_env(env, lambda: art.Decoder(dev["q"], dev["k_pages"], dev["block_table"]))
        outs = []
        for i in range(4):
            out, stop = _with_env(env, lambda: dec(dev["q"], dev["k_pages"], dev["v_pages"], dev["block_table"],
                                                   dev["block_order"], dev["seq_lens"], case["eps_mag"],
                                                   case["eps_dir"], case["patience"]))
            torch.cuda.synchronize()
            ctrl = dec.workspace[:16].view(torch.int32).cpu().numpy()
            assert ctrl[0] == expect_epoch(i), ctrl   # stored epoch
            assert ctrl[1] == 0, ctrl                 # finished-workgroup counter back to 0
            assert ctrl[2] == 0, ctrl                 # no bounded wait ran out
            outs.append((out.cpu(), stop.cpu()))
        for o, s_ in outs[1:]:
            assert torch.equal(o, outs[0][0]) and torch.equal(s_, outs[0][1])
        return outs[0]

    lb = run(dict(ART_SCHED="lb"), lambda i: i + 1)
    wn = run(dict(ART_SCHED="win"), lambda i: 0)   # the windowed path uses no epoch-tagged words
    assert torch.equal(lb[0], wn[0]) and torch.equal(lb[1], wn[1])
    a = run(dict(ART_SCHED="scan", ART_HELPERS="64"), lambda i: i + 1)
    b = run(dict(ART_SCHED="scan", ART_HELPERS="0"), lambda i: 0)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


# ---- the look-back scheduler on every kernel variant and edge case ---------------------------------------
#
# ART_SCHED=auto sends only few, long streams to the look-back kernel; these run the shape corners and the
# edge cases through it explicitly.

@pytest.mark.parametrize("sched", ["lb", "win", "stream", "seg", "scan"])
@pytest.mark.parametrize("w", SHAPES, ids=[w.name for w in SHAPES])
def test_lookback_and_windowed_shape_matrix(w, sched):
    case = synth.make_case(w, batch=2, context=2000 + 9)
    print(f"[{sched} shape] {w.name}", flush=True)
    _with_env(dict(ART_SCHED=sched), lambda: check_art(case))


@pytest.mark.parametrize("env", [dict(ART_SCHED="lb", ART_WINDOW="2"), dict(ART_SCHED="win", ART_WIN_SPLIT="2"),
                                 dict(ART_SCHED="stream", ART_LA0="1", ART_LA_SHIFT="30"), dict(ART_SCHED="scan"),
                                 dict(ART_SCHED="seg", ART_SEG_WIN="1")],
                         ids=["lookback", "windowed", "stream", "scanners", "segments"])
def test_lookback_and_windowed_edge_cases(env):
    base = synth.make_case(W.LLAMA3_8B, batch=5, context=700)
    case = _with_lens(base, [0, 1, 15, 16, 17])
    _with_env(env, lambda: check_art(case, patience=1, eps_mag=0.5, eps_dir=0.5))
    _with_env(env, lambda: check_art(case))
    out, stop, fetched = _with_env(env, lambda: _device_run(case, 1e-3, 1e-4, 4))
    assert np.all(out[0] == 0.0) and np.all(stop[0] == 0) and np.all(fetched[0] == 0)

    case = synth.make_case(W.LLAMA3_8B, batch=3, context=3000)
    rng = np.random.default_rng(11)
    n = int(_nblocks(case)[0])
    order = case["block_order"].copy()
    order[0, :n] = list(range(n - 1, -1, -1))  # block 0 last: nobody can stop early
    order[1, :n] = rng.permutation(n)
    order[2, :n] = [5, 4, 3, 2, 1, 0] + list(range(6, n))
    case["block_order"] = order
    rep, out, stop, fetched = _with_env(env, lambda: check_art(case, eps_mag=1e-2, eps_dir=1e-3, patience=2))
    assert np.all(stop[0] == n)

    case = synth.make_case(W.LLAMA3_8B, batch=2, context=4096)
    rep, out, stop, fetched = _with_env(env, lambda: check_art(case, eps_mag=10.0, eps_dir=10.0, patience=1))
    assert np.all(stop == 2)
    _with_env(env, lambda: check_art(case, eps_mag=10.0, eps_dir=10.0, patience=5))
    # a patience no head can reach: every head runs to its end
    rep, out, stop, fetched = _with_env(env, lambda: check_art(case, eps_mag=10.0, eps_dir=10.0, patience=3000))
    assert np.all(stop == _nblocks(case)[:, None])
    from kv_cache_run_amd import art

    dev = art.case_to_device(case)
    desc = art.make_desc(dev["q"], dev["k_pages"], dev["block_table"])
    if env["ART_SCHED"] == "lb":
        # patience above what the look-back records hold: that call ran the scanners, same contract
        assert _with_env(env, lambda: art.art_decode_kernel_choice(desc, 1e-3, 1e-4, 3000)) == art.ART_KERNEL_SCANNERS
        assert _with_env(env, lambda: art.art_decode_kernel_choice(desc, 1e-3, 1e-4, 30)) == art.ART_KERNEL_LOOKBACK
    else:
        want = {"win": art.ART_KERNEL_WINDOWED, "stream": art.ART_KERNEL_STREAM, "scan": art.ART_KERNEL_SCANNERS,
                "seg": art.ART_KERNEL_SEGMENTS}
        assert _with_env(env, lambda: art.art_decode_kernel_choice(desc, 1e-3, 1e-4, 3000)) == want[env["ART_SCHED"]]


# ---- detector ablation: one test switched off (threshold +inf) or patience 1 -----------------------------

ABLATION_VARIANTS = {"scale_only": (None, math.inf, None), "direction_only": (math.inf, None, None),
                     "patience_1": (None, None, 1), "both_off": (math.inf, math.inf, None)}


@pytest.mark.parametrize("variant", list(ABLATION_VARIANTS), ids=list(ABLATION_VARIANTS))
@pytest.mark.parametrize("w", [W.HEAVY_TAIL, W.VALUE_HEAVY, W.RECENT], ids=["heavytail", "valueheavy", "recent"])
def test_ablation_variants_parity(w, variant):
    case = synth.make_case(w, batch=2, context=4096 - 5)
    em, ed, p = ABLATION_VARIANTS[variant]
    check_art(case, eps_mag=em, eps_dir=ed, patience=p)


@pytest.mark.parametrize("sched", ["lb", "win", "stream", "seg"])
def test_ablation_through_lookback_and_windowed(sched):
    case = synth.make_case(W.VALUE_HEAVY, batch=2, context=4096 - 5)
    _with_env(dict(ART_SCHED=sched), lambda: check_art(case, eps_dir=math.inf))
    _with_env(dict(ART_SCHED=sched), lambda: check_art(case, eps_mag=math.inf, patience=1))


# ---- ART over a pruned cache: only the first visit_lens[s] entries of the order are visited ------------

def _pruned_case():
    """Block 0 plus a recent window (the default order's first entries), a random subset in random order with
    block 0 inside, one without block 0, an empty subset, a single block and the whole sequence."""
    case = synth.make_case(W.LLAMA3_8B, batch=6, context=3000 - 7)
    rng = np.random.default_rng(21)
    n = int(_nblocks(case)[0])
    order = case["block_order"].copy()
    vl = np.zeros(6, np.int32)
    vl[0] = 1 + 24                                       # sink + 24 newest blocks
    perm = rng.permutation(n)
    order[1, :n] = perm
    vl[1] = int(np.where(perm == 0)[0][0]) + 40          # random subset that holds block 0
    order[2, :n] = list(range(n - 1, -1, -1))            # block 0 last ...
    vl[2] = n // 2                                       # ... and not visited: no early stop
    vl[3] = 0
    vl[4] = 1
    vl[5] = n
    case["block_order"] = order
    case["visit_lens"] = vl
    return case


@pytest.mark.parametrize("sched", ["scan", "lb", "win", "stream", "seg"])
def test_pruned_cache_parity(sched):
    case = _pruned_case()
    print(f"[pruned] {sched}", flush=True)
    rep, out, stop, fetched = _with_env(dict(ART_SCHED=sched), lambda: check_art(case))
    n = _nblocks(case)
    assert np.all(stop[2] == n[2])          # no block 0 among the visited blocks
    assert np.all(stop[3] == 0) and np.all(out[3] == 0.0) and np.all(fetched[3] == 0)
    _with_env(dict(ART_SCHED=sched), lambda: check_art(case, eps_mag=0.5, eps_dir=0.5, patience=1))


def test_pruned_cache_full_attention():
    case = _pruned_case()
    check_full(case)
    ref_case = dict(case)
    ref_case["visit_lens"] = None
    a = _device_run(case, 0.0, 0.0, 1)
    b = _device_run(ref_case, 0.0, 0.0, 1)
    # the whole sequence visited (row 5) is the plain call, summed in visit order instead of logical order
    assert np.array_equal(a[1][5], b[1][5])
    assert oracle.feasible.max_rel_err(a[0][5], b[0][5]) <= 1e-5


# ---- probe-vector detector: the statistics over the leading P output coordinates -------------------------

@pytest.mark.parametrize("sched", ["scan", "lb", "win", "stream", "seg"])
@pytest.mark.parametrize("w,P", [(W.LLAMA3_8B, 8), (W.LLAMA3_8B, 32), (W.LLAMA3_8B, 64), (W.TINY, 16)],
                         ids=["llama-P8", "llama-P32", "llama-P64", "tiny-P16"])
def test_probe_vector_parity(w, P, sched):
    case = synth.make_case(w, batch=min(w.batch, 3), context=3000 - 11)
    case["probe"] = P
    case["probe_coords"] = np.arange(P)
    print(f"[probe] {w.name} P={P} {sched}", flush=True)
    _with_env(dict(ART_SCHED=sched), lambda: check_art(case))


def test_probe_of_every_coordinate_is_the_plain_detector():
    case = synth.make_case(W.LLAMA3_8B, batch=2, context=2000)
    a = _device_run(case, case["eps_mag"], case["eps_dir"], case["patience"])
    case["probe"] = case["head_dim"]
    b = _device_run(case, case["eps_mag"], case["eps_dir"], case["patience"])
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ---- importance-first order: key summaries and the order pre-pass, then ART on that order ---------------

def _device_order(case):
    import torch

    from kv_cache_run_amd import art

    dev = art.case_to_device(case)
    sm = art.block_key_summary(dev["q"], dev["k_pages"], dev["block_table"], dev["seq_lens"], k_scale=dev["k_scale"])
    order = art.importance_order(dev["q"], dev["k_pages"], sm, dev["block_table"], dev["seq_lens"])
    torch.cuda.synchronize()
    return sm.cpu().numpy().astype(np.float64), order.cpu().numpy()


def _oracle_scores(case, summary):
    return oracle.block_scores(case["q"], summary, case["block_table"], case["seq_lens"],
                               block_size=case["block_size"], num_kv_heads=case["num_kv_heads"],
                               q_dtype=case["q_dtype"])


@pytest.mark.parametrize("w", [W.TINY, W.LLAMA3_8B, W.QWEN_FP8, W.RAGGED], ids=["f32", "bf16", "fp8", "ragged"])
def test_importance_order_parity(w):
    case = synth.make_case(w, batch=min(w.batch, 3), context=(700, 3000) if isinstance(w.context, tuple) else 2500 - 3)
    print(f"[order] {w.name}", flush=True)
    sm, order = _device_order(case)
    ref_sm = oracle.block_key_summary(case["k_pages"], case["block_table"], case["seq_lens"],
                                      block_size=case["block_size"], num_kv_heads=case["num_kv_heads"],
                                      kv_dtype=case["kv_dtype"], k_scale=case["k_scale"])
    used = np.unique(np.concatenate([case["block_table"][s, :n] for s, n in enumerate(_nblocks(case))]))
    assert np.allclose(sm[used], ref_sm[used], rtol=1e-5, atol=1e-6)
    sc = _oracle_scores(case, ref_sm)
    ref = oracle.importance_order(sc, case["seq_lens"], block_size=case["block_size"])
    for s, n in enumerate(_nblocks(case)):
        o = order[s, :n]
        assert o[0] == 0 and np.array_equal(np.sort(o), np.arange(n))
        # the same descending score sequence; the blocks may swap only where scores agree to float32 rounding
        a, b = sc[s, o[1:]], sc[s, ref[s, 1:n]]
        tol = 1e-5 * max(1.0, float(np.abs(sc[s, :n]).max()))
        assert np.all(np.abs(a - b) <= tol)
        assert np.all(np.diff(a) <= tol)


def test_importance_order_with_equal_scores_is_recency_first():
    case = synth.make_case(W.LLAMA3_8B, batch=2, context=1500)
    case["k_pages"] = np.zeros_like(case["k_pages"])   # every summary 0: every score ties
    sm, order = _device_order(case)
    for s, n in enumerate(_nblocks(case)):
        assert list(order[s, :n]) == [0] + list(range(n - 1, 0, -1))


@pytest.mark.parametrize("sched", ["scan", "lb", "win", "stream", "seg"])
def test_art_on_the_importance_order(sched):
    case = synth.make_case(W.LLAMA3_8B, batch=3, context=3000 - 5)
    _, order = _device_order(case)
    case["block_order"] = order.astype(np.int32)
    _with_env(dict(ART_SCHED=sched), lambda: check_art(case))


def test_skip_statistics_flag_gives_full_attention_in_every_scheduler():
    """ART_FLAG_SKIP_STATS (a measurement flag) folds every block with no test passing: the result is the
    terminating kernel's full attention, whatever the thresholds, through every scheduler."""
    from kv_cache_run_amd import art

    case = synth.make_case(W.LLAMA3_8B, batch=2, context=1500)
    ref = _device_run(case, 0.0, 0.0, 4, flags=art.ART_FLAG_KEEP_DETECTOR)
    n = _nblocks(case)
    for sched in ("scan", "lb", "win", "stream", "seg"):
        out, stop, fetched = _with_env(dict(ART_SCHED=sched),
                                       lambda: _device_run(case, 1e-3, 1e-4, 4, flags=art.ART_FLAG_SKIP_STATS))
        assert np.all(stop == n[:, None]), sched
        assert oracle.feasible.max_rel_err(out, ref[0]) <= 1e-5, sched


def test_importance_order_on_degenerate_lengths():
    """Empty, one-token, one-block, block-boundary and longer sequences: the pre-pass writes a valid order
    (block 0 first) of exactly n_s entries, with the oracle's score sequence; ART then runs on it."""
    base = synth.make_case(W.LLAMA3_8B, batch=6, context=1000)
    case = _with_lens(base, [0, 1, 16, 17, 250, 1000])
    sm, order = _device_order(case)
    ref_sm = oracle.block_key_summary(case["k_pages"], case["block_table"], case["seq_lens"],
                                      block_size=case["block_size"], num_kv_heads=case["num_kv_heads"],
                                      kv_dtype=case["kv_dtype"], k_scale=case["k_scale"])
    sc = _oracle_scores(case, ref_sm)
    ref = oracle.importance_order(sc, case["seq_lens"], block_size=case["block_size"])
    for s, n in enumerate(_nblocks(case)):
        assert np.all(order[s, n:] == -1)          # positions past n_s untouched
        if n == 0:
            continue
        o = order[s, :n]
        assert o[0] == 0 and np.array_equal(np.sort(o), np.arange(n))
        tol = 1e-5 * max(1.0, float(np.abs(sc[s, :n]).max()))
        assert np.all(np.abs(sc[s, o[1:]] - sc[s, ref[s, 1:n]]) <= tol)
    case["block_order"] = order.astype(np.int32)
    check_art(case)


# ---- seeded random configurations: features combined across the supported matrix ----------------------

def _random_case(seed):
    rng = np.random.default_rng(1000 + seed)
    D = int(rng.choice([64, 128]))
    B = int(rng.choice([16, 32]))
    hkv = int(rng.choice([1, 2, 4]))
    g = int(rng.choice([1, 3, 4, 7, 8, 16]))
    kv = str(rng.choice(["f32", "bf16", "fp8_e4m3fn"]))
    q = "f32" if kv == "f32" else "bf16"
    batch = int(rng.integers(1, 4))
    w = W.LLAMA3_8B.scaled(name=f"random-{seed}", batch=batch, num_q_heads=hkv * g, num_kv_heads=hkv, head_dim=D,
                           block_size=B, q_dtype=q, kv_dtype=kv, context=(1, 40 * B),
                           heavy=("frac", float(rng.uniform(0.0, 0.08))), seed=2000 + seed)
    case = synth.make_case(w)
    lens = case["seq_lens"].copy()
    lens[0] = int(rng.choice([0, 1, B, B + 1, lens[0]]))   # a degenerate first sequence now and then
    case = _with_lens(case, lens)
    n = _nblocks(case)
    order = case["block_order"].copy()
    for s in range(batch):
        kind = int(rng.integers(0, 3))
        if n[s] > 1 and kind == 1:      # random order
            order[s, :n[s]] = rng.permutation(n[s])
        elif n[s] > 1 and kind == 2:    # block 0 last
            order[s, :n[s]] = list(range(n[s] - 1, -1, -1))
    case["block_order"] = order
    if rng.random() < 0.3:
        case["visit_lens"] = np.array([int(rng.integers(0, m + 1)) for m in n], dtype=np.int32)
    if rng.random() < 0.3:
        P = int(rng.choice([8, 16, D // 2]))
        case["probe"], case["probe_coords"] = P, np.arange(P)
    em = float(10 ** rng.uniform(-4, -1))
    ed = float(10 ** rng.uniform(-5, -2))
    p = int(rng.integers(1, 7))
    sched = str(rng.choice(["scan", "lb", "win", "auto", "stream", "seg"]))
    return case, em, ed, p, sched


@pytest.mark.parametrize("seed", range(12))
def test_random_configurations(seed):
    case, em, ed, p, sched = _random_case(seed)
    print(f"[random {seed}] D={case['head_dim']} B={case['block_size']} Hq={case['num_q_heads']} "
          f"Hkv={case['num_kv_heads']} {case['kv_dtype']} lens={list(case['seq_lens'])} sched={sched} "
          f"visits={case.get('visit_lens')} probe={case.get('probe')} eps=({em:.2e},{ed:.2e}) p={p}", flush=True)
    _with_env(dict(ART_SCHED=sched), lambda: check_art(case, eps_mag=em, eps_dir=ed, patience=p))


# ---- the input-contract check (art_check_inputs) -------------------------------------------------------

_TORCH_DT = {"bf16": "bfloat16", "fp8_e4m3fn": "float8_e4m3fn", "f32": "float32"}


def _check_dev(case, bt, bo, sl, vl=None, num_pages=None):
    """art_check_inputs on device copies of the integer tables (q and the pages enter only through their
    shapes and dtypes, so they are meta tensors)."""
    import torch

    from kv_cache_run_amd import art

    pages = case["k_pages"].shape[0] if num_pages is None else num_pages
    q = torch.empty(case["q"].shape, dtype=getattr(torch, _TORCH_DT[case["q_dtype"]]), device="meta")
    kp = torch.empty((pages,) + tuple(case["k_pages"].shape[1:]), dtype=getattr(torch, _TORCH_DT[case["kv_dtype"]]),
                     device="meta")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    r = art.check_inputs(q, kp, t(bt), t(bo), t(sl), visit_lens=None if vl is None else t(vl))
    torch.cuda.synchronize()
    return tuple(int(x) for x in r.cpu())


def _corrupt(case, rng):
    """1-3 planted violations of random kinds at random places (and sometimes a visit count per sequence)."""
    bt, bo, sl = case["block_table"].copy(), case["block_order"].copy(), case["seq_lens"].copy()
    batch, mb = bo.shape
    B = case["block_size"]
    pages = case["k_pages"].shape[0]
    n = -(-sl.astype(np.int64) // B)
    for _ in range(int(rng.integers(1, 4))):
        s = int(rng.integers(0, batch))
        kind = int(rng.integers(0, 6))
        if kind == 0:
            sl[s] = int(rng.choice([-1, -int(rng.integers(2, 1 << 20)), mb * B + 1, mb * B + int(rng.integers(2, 999))]))
        elif n[s] >= 2:
            t, u = (int(x) for x in rng.choice(n[s], size=2, replace=False))
            if kind == 1:
                bo[s, u] = int(rng.choice([-1, n[s], n[s] + int(rng.integers(0, 99)), -(1 << 30)]))
            elif kind == 2:
                bo[s, u] = bo[s, t]
            elif kind == 3:
                b = bo[s, u]
                if 0 <= b < n[s]:
                    bt[s, b] = int(rng.choice([pages, pages + int(rng.integers(0, 99)), -1]))
            elif kind == 4:
                bo[s, u], bo[s, t] = bo[s, t], bo[s, u]  # still valid
            else:
                bt[s, mb - 1] = -5  # a cell no visit reaches when n_s < max_blocks
    vl = None
    if rng.random() < 0.3:
        vl = np.array([int(rng.integers(-2, m + 3)) for m in n], dtype=np.int32)
    return bt, bo, sl, vl


@pytest.mark.parametrize("w,kw", REDUCED, ids=[f"{w.name}-{kw}" for w, kw in REDUCED])
def test_check_inputs_matches_the_oracle(w, kw):
    case = synth.make_case(w, **kw)
    pages = case["k_pages"].shape[0]
    args = (case["block_table"], case["block_order"], case["seq_lens"])
    print(f"[check] {case['workload']}", flush=True)
    assert _check_dev(case, *args) == (0, 0, 0, 0)
    rng = np.random.default_rng(zlib.crc32(case["workload"].encode()))
    codes = set()
    for trial in range(24):
        bt, bo, sl, vl = _corrupt(case, rng)
        want = oracle.check_inputs(bt, bo, sl, num_pages=pages, block_size=case["block_size"], visit_lens=vl)
        got = _check_dev(case, bt, bo, sl, vl)
        assert got == want, (trial, got, want)
        codes.add(want[0])
    assert len(codes) >= 3, codes


def test_check_inputs_at_the_longest_rows():
    """Rows of 2^18 blocks (the largest the check takes), one at full capacity: valid, then a repeat and a bad
    page near the end of the row, and an entry out of range in the second sequence."""
    base = synth.make_case(W.TINY, batch=2, context=64)
    mb, B = 1 << 18, base["block_size"]
    rng = np.random.default_rng(3)
    pages = 1 << 20
    bt = rng.integers(0, pages, size=(2, mb)).astype(np.int32)
    bo = np.full((2, mb), -1, dtype=np.int32)
    bo[0] = np.concatenate([[0], rng.permutation(np.arange(1, mb))])
    n1 = 100000
    bo[1, :n1] = rng.permutation(n1)
    sl = np.array([mb * B, n1 * B - 3], dtype=np.int32)
    case = dict(base, block_size=B)
    assert _check_dev(case, bt, bo, sl, num_pages=pages) == (0, 0, 0, 0)
    bo2 = bo.copy()
    bo2[0, 262000] = bo2[0, 200000]
    bt2 = bt.copy()
    bt2[0, bo[0, 150000]] = pages
    bo2[1, 5] = n1
    for a in ((bt, bo2, sl), (bt2, bo, sl), (bt2, bo2, sl), (bt, bo2, sl[::-1].copy())):
        want = oracle.check_inputs(*a, num_pages=pages, block_size=B)
        assert _check_dev(case, *a, num_pages=pages) == want, want
    assert oracle.check_inputs(bt, bo2, sl, num_pages=pages, block_size=B) == (3, 0, 200000, int(bo[0, 200000]))


def test_decoder_checks_inputs_when_asked():
    import torch

    from kv_cache_run_amd import art

    case = synth.make_case(W.TINY)
    dev = art.case_to_device(case)
    dec = art.Decoder(dev["q"], dev["k_pages"], dev["block_table"], check_inputs=True)
    out, stop = dec(dev["q"], dev["k_pages"], dev["v_pages"], dev["block_table"], dev["block_order"], dev["seq_lens"],
                    case["eps_mag"], case["eps_dir"], case["patience"])
    torch.cuda.synchronize()
    ref = _device_run(case, case["eps_mag"], case["eps_dir"], case["patience"])
    assert np.array_equal(out.cpu().numpy().astype(np.float64), ref[0]) and np.array_equal(stop.cpu().numpy(), ref[1])
    bad = dev["block_order"].clone()
    bad[0, 3] = bad[0, 1]
    with pytest.raises(ValueError, match="repeated"):
        dec(dev["q"], dev["k_pages"], dev["v_pages"], dev["block_table"], bad, dev["seq_lens"], case["eps_mag"],
            case["eps_dir"], case["patience"])


@pytest.mark.parametrize("w", [W.LLAMA3_8B, W.QWEN_FP8], ids=["bf16", "fp8"])
@pytest.mark.parametrize("sched", ["scan", "lb", "win", "stream", "seg", "full"])
def test_pages_past_4_gib(sched, w):
    """Page addressing is 64-bit: the same pages (and fp8 scales) placed past 4 GiB of K and of V (a pool
    of ≈4.3 GiB each) give the same bits as at low page ids, for each ART scheduler and for full attention."""
    import torch

    from kv_cache_run_amd import art

    case = synth.make_case(w, batch=2, context=3000)
    dev = art.case_to_device(case)
    k, v = dev["k_pages"], dev["v_pages"]
    page_bytes = k[0].numel() * k.element_size()
    base = (4 << 30) // page_bytes + 1000
    kb = torch.empty((base + k.shape[0],) + tuple(k.shape[1:]), dtype=k.dtype, device=k.device)
    vb = torch.empty_like(kb)
    kb[base:] = k
    vb[base:] = v
    scales = {}
    if dev["k_scale"] is not None:
        for name in ("k_scale", "v_scale"):
            sc = torch.ones((base + k.shape[0], k.shape[1]), dtype=torch.float32, device=k.device)
            sc[base:] = dev[name]
            scales[name] = sc
    bt = dev["block_table"] + base
    assert (int(bt.min()) * page_bytes) >= (4 << 30)
    em, ed, p = (0.0, 0.0, 1) if sched == "full" else (case["eps_mag"], case["eps_dir"], case["patience"])
    env = {} if sched == "full" else dict(ART_SCHED=sched)
    print(f"[4gib] {sched} pool {kb.shape[0]} pages ({kb.numel() * kb.element_size() >> 20} MiB each for K and V)",
          flush=True)

    def run(kp, vp, table, ks, vs):
        dec = art.Decoder(dev["q"], kp, table)
        out, stop = dec(dev["q"], kp, vp, table, dev["block_order"], dev["seq_lens"], em, ed, p, k_scale=ks,
                        v_scale=vs)
        torch.cuda.synchronize()
        return out.cpu().numpy(), stop.cpu().numpy()

    lo = _with_env(env, lambda: run(k, v, dev["block_table"], dev["k_scale"], dev["v_scale"]))
    hi = _with_env(env, lambda: run(kb, vb, bt, scales.get("k_scale"), scales.get("v_scale")))
    assert np.array_equal(lo[0], hi[0]) and np.array_equal(lo[1], hi[1])
    del kb, vb
    torch.cuda.empty_cache()


# ---- bounded waits that give up: forced from the host with the smallest spin limit -----------------------


@pytest.mark.parametrize("sched", ["lb", "stream", "seg", "scan-helpers"])
def test_bounded_waits_that_give_up_are_reported(sched):
    """ART_SPIN_LIMIT=1 (two polls) makes waits between workgroups or waves give up; every wait is bounded, so
    every kernel still exits.  A head whose result a give-up touched reads stop -1 or NaN output
    (two workgroups of the look-back kernel may both write one head, so the two marks can mix); every other
    head passes the oracle check, and any give-up sets the workspace's failure word."""
    from kv_cache_run_amd import art

    env = {"lb": dict(ART_SCHED="lb", ART_SPIN_LIMIT="1"), "stream": dict(ART_SCHED="stream", ART_SPIN_LIMIT="1"),
           "seg": dict(ART_SCHED="seg", ART_SPIN_LIMIT="1"),
           "scan-helpers": dict(ART_SCHED="scan", ART_HELPERS="256", ART_SPIN_LIMIT="1")}[sched]
    case = synth.make_case(W.RAGGED, batch=4)

    def run():
        import torch

        dev = art.case_to_device(case)
        dec = art.Decoder(dev["q"], dev["k_pages"], dev["block_table"])
        art.art_decode_workspace_init(dec.workspace) if dec.workspace is not None else None
        assert dec.workspace is None or not art.art_decode_workspace_status(dec.workspace)
        out, stop = dec(dev["q"], dev["k_pages"], dev["v_pages"], dev["block_table"], dev["block_order"],
                        dev["seq_lens"], case["eps_mag"], case["eps_dir"], case["patience"])
        torch.cuda.synchronize()
        failed = None if dec.workspace is None else art.art_decode_workspace_status(dec.workspace)
        return out.cpu().numpy().astype(np.float64), stop.cpu().numpy(), failed

    out, stop, failed = _with_env(env, run)
    gave_up = (stop == -1) | np.isnan(out).any(axis=-1)
    print(f"[give-up] {sched}: {int(gave_up.sum())} of {stop.size} heads gave up; status {failed}", flush=True)
    if gave_up.any():
        assert failed is True
    if sched == "stream":
        # the detectors' first wait (two polls) ends long before eight blocks' tiles can arrive
        assert gave_up.any() and failed is True
    ok = [(s, h) for s in range(case["batch"]) for h in range(case["num_q_heads"]) if not gave_up[s, h]]
    if ok:
        ref = oracle.art_reference(*synth.oracle_arrays(case), eps_mag=case["eps_mag"], eps_dir=case["eps_dir"],
                                   patience=case["patience"], pairs=ok, **synth.oracle_kwargs(case),
                                   **synth.oracle_detector_kwargs(case))
        rep = oracle.compare_with_oracle(out, stop, case, ref, eps_mag=case["eps_mag"], eps_dir=case["eps_dir"],
                                         patience=case["patience"], pairs=ok)
        assert rep["bad"] == [] and rep["max_rel_err"] <= TOL, rep
