"""Benchmark: ART paged decode attention on one MI355X.

One step = one ``art_decode`` call over the whole batch (one decode step of
one attention layer).  The headline is the ragged long-batch decode (batch 32,
32 q heads / 8 kv heads, D=128, bf16 K/V, context U(4096, 32768) per
sequence, KV block 16): the largest of the workloads, 2.27 GB of KV.  Prints
one JSON line.

Timing: inputs are resident in HBM before the timed region.  To keep the
256 MB MALL and the L2s cold without a flush kernel inside the timed region,
the page pool holds R copies of the cache and consecutive calls use block
tables that point into different copies (R chosen so that R-1 calls read more
than 512 MB).  The K timed calls are captured into one HIP graph (so host
launch overhead cannot gap the few-µs kernels) and replayed back to back on
the current stream between two HIP events; µs/step = elapsed / K.  The same K
calls launched eagerly from Python (ctypes, no graph) are timed as well.

Also reported: full-attention mode, the fraction of KV blocks the kernel read
(its own counter), the floor for that fraction from the kernel's own stops,
achieved bandwidth on algorithmic and on actually-read bytes, every other
workload in both modes, threshold sweeps (step time against the KV fraction
read), and the CPU oracle timed on the host.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

PEAK_GBPS = 8000.0
METRIC = "decode-attn µs/step + achieved HBM GB/s (frac of peak) + KV fraction read, 1 GPU"
KERNEL_SOURCES = ["kv_cache_run_amd/csrc/art_kernels_impl.h", "kv_cache_run_amd/csrc/art_stream.h",
                  "kv_cache_run_amd/csrc/art_seg.h", "kv_cache_run_amd/csrc/art_internal.h", "kv_cache_run_amd/csrc/kern_art_bf16.hip",
                  "kv_cache_run_amd/csrc/kern_art_fp8.hip", "kv_cache_run_amd/csrc/kern_art_f32.hip",
                  "kv_cache_run_amd/csrc/kern_full_bf16.hip", "kv_cache_run_amd/csrc/kern_full_fp8.hip",
                  "kv_cache_run_amd/csrc/kern_full_f32.hip", "kv_cache_run_amd/csrc/art_api.cpp"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(case: dict, stop: np.ndarray) -> dict:
    """Bytes the method itself must move for one call, given the heads' stops.

    Per stream (sequence, kv-head): F = max over the query group of stop_block
    blocks of K and V tiles (plus two fp32 scales per tile for fp8); per
    sequence: the order and table entries of its longest-running stream;
    plus q, seq_lens, out and stop_block.
    """
    B, D = case["block_size"], case["head_dim"]
    es = {"f32": 4, "bf16": 2, "fp8_e4m3fn": 1}[case["kv_dtype"]]
    qes = {"f32": 4, "bf16": 2}[case["q_dtype"]]
    tile = 2 * B * D * es + (8 if case["kv_dtype"] == "fp8_e4m3fn" else 0)
    g = case["num_q_heads"] // case["num_kv_heads"]
    F = stop.reshape(case["batch"], case["num_kv_heads"], g).max(axis=2).astype(np.int64)
    kv = int(F.sum()) * tile
    meta = int(F.max(axis=1).sum()) * 8 + case["batch"] * 4
    q = case["batch"] * case["num_q_heads"] * D * qes
    outb = case["batch"] * case["num_q_heads"] * (D * 4 + 4)
    return {"total": kv + meta + q + outb, "kv": kv, "blocks": int(F.sum()), "tile": tile}


_CPU_CASE = None  # the case the oracle workers read (inherited through fork, never pickled)


def _oracle_worker(args):
    """Run the oracle on one stream (sequence, kv-head): all its query heads; returns the wall seconds."""
    (s, kvh, mode) = args
    case = _CPU_CASE
    import oracle
    from kv_cache_run_amd import synth

    g = case["num_q_heads"] // case["num_kv_heads"]
    pairs = [(s, kvh * g + j) for j in range(g)]
    t = time.perf_counter()
    if mode == "art":
        oracle.art_reference(*synth.oracle_arrays(case), eps_mag=case["eps_mag"], eps_dir=case["eps_dir"],
                             patience=case["patience"], pairs=pairs, **synth.oracle_kwargs(case))
    else:
        oracle.art_reference(*synth.oracle_arrays(case), eps_mag=0.0, eps_dir=0.0, patience=1, pairs=pairs,
                             **synth.oracle_kwargs(case))
    return time.perf_counter() - t


def cpu_baseline(case: dict, max_seconds: float = 10.0) -> dict:
    """Time the float64 oracle as it stands on the host, in ART and in full-attention mode.

    Work items are streams (sequence, kv-head) with all their query heads: the oracle decodes a stream's
    blocks once for its heads.  Per mode, a seeded random order of the streams is run (a) on one core, item
    by item until the batch is done or ``max_seconds`` have passed, and (b) on a pool of one single-threaded
    worker process per core, at most 16 (the host share of one GPU on the box), over as many items as the
    one-core rate says fit in ``max_seconds`` of wall time.  A partial sample is scaled to the whole batch
    by the fraction of streams it covered.  Must run before the GPU is initialised (the pool forks).
    """
    import multiprocessing as mp

    global _CPU_CASE
    _CPU_CASE = case
    for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[k] = "1"
    host_cores = len(os.sched_getaffinity(0))
    workers = max(1, min(16, host_cores))
    items = [(s, k) for s in range(case["batch"]) for k in range(case["num_kv_heads"])]
    rng = np.random.default_rng(0)
    items = [items[i] for i in rng.permutation(len(items))]
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    res = {"host_cores": host_cores, "cpu_model": model}
    ctx = mp.get_context("fork")
    for mode in ("art", "full"):
        t0 = time.perf_counter()
        done1 = 0
        for s, k in items:
            _oracle_worker((s, k, mode))
            done1 += 1
            if time.perf_counter() - t0 > max_seconds:
                break
        wall1 = time.perf_counter() - t0
        us1 = wall1 * 1e6 * len(items) / done1
        per_item = wall1 / done1
        nwant = int(min(len(items), max(workers, math.floor(max_seconds * workers / max(per_item, 1e-9)))))
        jobs = [(s, k, mode) for s, k in items[:nwant]]
        t0 = time.perf_counter()
        with ctx.Pool(workers) as pool:
            pool.map(_oracle_worker, jobs, chunksize=1)
        walln = time.perf_counter() - t0
        res[mode] = {"us_per_step": walln * 1e6 * len(items) / nwant, "cores": workers,
                     "streams_timed": nwant, "wall_s": walln,
                     "one_core_us_per_step": us1, "one_core_streams_timed": done1, "one_core_wall_s": wall1}
    res["streams"] = len(items)
    return res


def read_traffic(kernel: str, workload: str) -> dict | None:
    """HBM traffic from the committed counter summary, if it matches the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"{kernel}--{workload}--counters.md")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if line.startswith("- ") and ":" in line:
                k, v = line[2:].split(":", 1)
                vals[k.strip()] = v.strip().strip("`")
    if vals.get("kernel_source_hash") != kernel_source_hash():
        return None
    try:
        return {"bytes_per_launch": float(vals["hbm_bytes_per_launch"])}
    except (KeyError, ValueError):
        return None


# A "setting" is (thresholds, patience, flags).  One reference call learns
# the work (stops, tiles read); then K calls are captured into one HIP
# graph over rotating page-pool copies and replayed between two events.
def time_setting(case, dev, em, ed, patience, flags, steps, warmup, outputs=False, visit_lens=None):
    import torch

    from kv_cache_run_amd import art

    stream = torch.cuda.current_stream()
    B = case["block_size"]
    n = (case["seq_lens"].astype(np.int64) + B - 1) // B
    total_blocks = int(n.sum()) * case["num_kv_heads"]
    kv_tile = 2 * B * case["head_dim"] * {"f32": 4, "bf16": 2, "fp8_e4m3fn": 1}[case["kv_dtype"]]
    pool_bytes = case["k_pages"].nbytes + case["v_pages"].nbytes
    out = torch.empty((case["batch"], case["num_q_heads"], case["head_dim"]), dtype=torch.float32,
                      device="cuda")
    stop = torch.empty((case["batch"], case["num_q_heads"]), dtype=torch.int32, device="cuda")
    fetched = torch.empty((case["batch"], case["num_kv_heads"]), dtype=torch.int32, device="cuda")

    def one_call(table, dec, kp, vp, ks, vs):
        dec(dev["q"], kp, vp, table, dev["block_order"], dev["seq_lens"], em, ed, patience, k_scale=ks,
            v_scale=vs, out=out, stop_block=stop, blocks_fetched=fetched, flags=flags, visit_lens=visit_lens)

    dec = art.Decoder(dev["q"], dev["k_pages"], dev["block_table"])
    one_call(dev["block_table"], dec, dev["k_pages"], dev["v_pages"], dev["k_scale"], dev["v_scale"])
    torch.cuda.synchronize()
    stop_h = stop.cpu().numpy()
    fetched_h = fetched.cpu().numpy()
    out_h = out.cpu().numpy() if outputs else None
    read_bytes = int(fetched_h.sum()) * kv_tile
    # page-pool copies so that consecutive calls read cold memory
    R = int(min(64, max(2, math.ceil(512e6 / max(read_bytes, 1)) + 1),
                max(2, (48 << 30) // max(pool_bytes, 1))))

    def rep(t):
        if t.dtype == torch.float8_e4m3fn:
            return t.view(torch.uint8).repeat(R, 1, 1, 1).view(torch.float8_e4m3fn)
        return t.repeat(R, 1, 1, 1)

    kp = rep(dev["k_pages"])
    vp = rep(dev["v_pages"])
    ks = None if dev["k_scale"] is None else dev["k_scale"].repeat(R, 1)
    vs = None if dev["v_scale"] is None else dev["v_scale"].repeat(R, 1)
    npages = case["num_pages"]
    tables = [dev["block_table"] + r * npages for r in range(R)]
    dec = art.Decoder(dev["q"], kp, dev["block_table"])
    for i in range(warmup):
        one_call(tables[i % R], dec, kp, vp, ks, vs)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(steps):
            one_call(tables[(warmup + i) % R], dec, kp, vp, ks, vs)
    graph.replay()  # first replay uploads the graph; untimed
    torch.cuda.synchronize()
    out_first = out.clone()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    graph.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / steps
    assert np.array_equal(stop.cpu().numpy(), stop_h), "stops changed across page copies / replays"
    assert torch.equal(out, out_first), "graph replays disagree"
    # the same calls launched eagerly from Python (ctypes per call, no graph)
    torch.cuda.synchronize()
    ev0.record(stream)
    for i in range(steps):
        one_call(tables[(warmup + i) % R], dec, kp, vp, ks, vs)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_eager = ev0.elapsed_time(ev1) / steps
    del graph, kp, vp, ks, vs, tables, dec
    torch.cuda.empty_cache()
    alg = algorithmic_bytes(case, stop_h)
    us = ms * 1e3
    res = {
        "us_per_step": us,
        "us_per_step_eager": ms_eager * 1e3,
        "wall_s": wall,
        "page_copies": R,
        "alg_bytes": alg["total"],
        "read_bytes": read_bytes,
        "achieved_GBps": alg["total"] / (us * 1e-6) / 1e9,
        "read_GBps": read_bytes / (us * 1e-6) / 1e9,
        "kv_fraction_read": float(fetched_h.sum()) / total_blocks,
        "kv_fraction_needed": alg["blocks"] / total_blocks,
    }
    if outputs:
        res["out"], res["stop"] = out_h, stop_h
    return res


def importance(steps: int, warmup: int) -> dict:
    """Recency-first (the default order) against importance-first (block 0, then blocks by the largest
    q . mean-key score): ART step time, KV read, the output's error against full attention on the same
    inputs (all on the device), and the order pre-pass's own time (the key summary is cache-write work:
    timed apart)."""
    import torch

    from kv_cache_run_amd import art, synth, workloads

    res = {}
    for w in (workloads.LLAMA3_8B, workloads.RECENT, workloads.LONG, workloads.QWEN_FP8):
        case = synth.make_case(w)
        dev = art.case_to_device(case)
        em, ed, p = case["eps_mag"], case["eps_dir"], case["patience"]
        full = time_setting(case, dev, 0.0, 0.0, p, art.ART_FLAG_FULL, steps, warmup, outputs=True)
        ref = full["out"].astype(np.float64)
        nrm = np.maximum(np.linalg.norm(ref, axis=-1), 1e-30)

        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        sm = art.block_key_summary(dev["q"], dev["k_pages"], dev["block_table"], dev["seq_lens"],
                                   k_scale=dev["k_scale"])
        torch.cuda.synchronize()
        ev[0].record()   # timed on a second, warm call (the first loads the code object)
        art.block_key_summary(dev["q"], dev["k_pages"], dev["block_table"], dev["seq_lens"], k_scale=dev["k_scale"],
                              summary=sm)
        ev[1].record()
        desc = art.make_desc(dev["q"], dev["k_pages"], dev["block_table"])
        ows = torch.empty(max(1, art.load_library().art_importance_order_workspace_bytes(ctypes.byref(desc))),
                          dtype=torch.uint8, device="cuda")
        order = art.importance_order(dev["q"], dev["k_pages"], sm, dev["block_table"], dev["seq_lens"], workspace=ows)
        torch.cuda.synchronize()
        reps = 20
        ev[2].record()
        for _ in range(reps):
            art.importance_order(dev["q"], dev["k_pages"], sm, dev["block_table"], dev["seq_lens"], block_order=order,
                                 workspace=ows)
        ev[3].record()
        torch.cuda.synchronize()
        rows = {"summary_us": round(ev[0].elapsed_time(ev[1]) * 1e3, 2),
                "order_prepass_us": round(ev[2].elapsed_time(ev[3]) * 1e3 / reps, 2),
                "full_us_per_step": round(full["us_per_step"], 3)}
        for name, d in (("recency_first", dev), ("importance_first", dict(dev, block_order=order))):
            r = time_setting(case, d, em, ed, p, 0, steps, warmup, outputs=True)
            err = np.linalg.norm(r["out"].astype(np.float64) - ref, axis=-1) / nrm
            rows[name] = {"us_per_step": round(r["us_per_step"], 3),
                          "kv_fraction_read": round(r["kv_fraction_read"], 5),
                          "kv_fraction_needed": round(r["kv_fraction_needed"], 5),
                          "rel_err_vs_full_mean": float(f"{err.mean():.4g}"),
                          "rel_err_vs_full_p99": float(f"{np.percentile(err, 99):.4g}")}
        res[w.name] = rows
        del dev, sm, order
        torch.cuda.empty_cache()
    return res


def probe(case: dict, dev: dict, steps: int, warmup: int) -> dict:
    """Probe-vector detector over the leading P coordinates of the output: step time, the detector's cost
    (every block folded with the detector kept, against the full-attention path) and how far the stops move
    from the whole-vector detector's."""
    from kv_cache_run_amd import art

    em, ed, p = case["eps_mag"], case["eps_dir"], case["patience"]
    B = case["block_size"]
    n = (case["seq_lens"].astype(np.int64) + B - 1) // B
    D = case["head_dim"]
    ref = time_setting(case, dev, em, ed, p, 0, steps, warmup, outputs=True)
    res = {}
    for P in (8, 16, 32, 64, D):
        fl = art.art_flag_probe(P) if P < D else 0
        r = ref if P == D else time_setting(case, dev, em, ed, p, fl, steps, warmup, outputs=True)
        keep = time_setting(case, dev, 0.0, 0.0, p, art.ART_FLAG_KEEP_DETECTOR | fl, steps, warmup)
        moved = r["stop"] != ref["stop"]
        res[f"P{P}"] = {
            "us_per_step": round(r["us_per_step"], 3),
            "kv_fraction_read": round(r["kv_fraction_read"], 5),
            "all_blocks_with_detector_us": round(keep["us_per_step"], 3),
            "heads_with_other_stop": round(float(moved.mean()), 5),
            "stop_shift_mean_blocks": round(float((r["stop"] - ref["stop"]).mean()), 4),
            "stop_shift_mean_abs_over_n": round(float((np.abs(r["stop"] - ref["stop"]) / n[:, None]).mean()), 6),
        }
    return res


def pruned(case: dict, dev: dict, steps: int, warmup: int) -> dict:
    """ART over a pruned cache (the default order visits block 0, then newest to oldest, so its first 1 + w
    entries are block 0 plus a recent window of w blocks) against full attention over the same blocks."""
    import torch

    from kv_cache_run_amd import art

    B = case["block_size"]
    n = (case["seq_lens"].astype(np.int64) + B - 1) // B
    res = {}
    for frac in (4, 16):
        vl_h = np.minimum(n, 1 + np.maximum(1, n // frac)).astype(np.int32)
        vl = torch.from_numpy(vl_h).cuda()
        a = time_setting(case, dev, case["eps_mag"], case["eps_dir"], case["patience"], 0, steps, warmup,
                         visit_lens=vl)
        f = time_setting(case, dev, 0.0, 0.0, case["patience"], art.ART_FLAG_FULL, steps, warmup, visit_lens=vl)
        tot = int(n.sum()) * case["num_kv_heads"]
        res[f"sink_plus_newest_1_{frac}"] = {
            "visited_fraction": round(float(vl_h.sum()) * case["num_kv_heads"] / tot, 5),
            "art_us_per_step": round(a["us_per_step"], 3),
            "art_kv_fraction_read": round(a["kv_fraction_read"], 5),
            "full_over_subset_us_per_step": round(f["us_per_step"], 3),
            "full_over_subset_kv_fraction_read": round(f["kv_fraction_read"], 5),
        }
    return res


def ablation(steps: int, warmup: int) -> dict:
    """Detector ablation: per workload and variant, the step time, the KV fractions and the error of the
    output at the stop against full attention on the same inputs (both from the device).  A switched-off
    test is a threshold of +inf."""
    from kv_cache_run_amd import art, synth, workloads

    res = {}
    for w in workloads.ABLATION:
        case = synth.make_case(w)
        dev = art.case_to_device(case)
        em, ed, p = case["eps_mag"], case["eps_dir"], case["patience"]
        full = time_setting(case, dev, 0.0, 0.0, p, art.ART_FLAG_FULL, steps, warmup, outputs=True)
        ref = full["out"].astype(np.float64)
        nrm = np.linalg.norm(ref, axis=-1)
        n = (case["seq_lens"].astype(np.int64) + case["block_size"] - 1) // case["block_size"]
        rows = {"full": {"us_per_step": round(full["us_per_step"], 3)}}
        for name, (e1, e2, pp) in {"both": (em, ed, p), "scale_only": (em, math.inf, p),
                                   "direction_only": (math.inf, ed, p), "patience_1": (em, ed, 1)}.items():
            r = time_setting(case, dev, e1, e2, pp, 0, steps, warmup, outputs=True)
            err = np.linalg.norm(r["out"].astype(np.float64) - ref, axis=-1) / np.maximum(nrm, 1e-30)
            rows[name] = {
                "us_per_step": round(r["us_per_step"], 3),
                "kv_fraction_read": round(r["kv_fraction_read"], 5),
                "stop_fraction_mean": round(float((r["stop"] / n[:, None]).mean()), 5),
                "rel_err_vs_full_mean": float(f"{err.mean():.4g}"),
                "rel_err_vs_full_p99": float(f"{np.percentile(err, 99):.4g}"),
                "rel_err_vs_full_max": float(f"{err.max():.4g}"),
            }
        res[w.name] = rows
        del dev
    return res


def sweep(case, dev, res_art, steps) -> dict:
    """Step time against the KV fraction read: thresholds scaled by 1/4 .. 4 at fixed patience, with a
    least-squares line through the points."""
    em0, ed0, p0 = case["eps_mag"], case["eps_dir"], case["patience"]
    pts = []
    for f in (0.25, 0.5, 1.0, 2.0, 4.0):
        r = res_art if f == 1.0 else time_setting(case, dev, em0 * f, ed0 * f, p0, 0, steps, 2)
        pts.append({"eps_scale": f, "kv_fraction_read": round(r["kv_fraction_read"], 5),
                    "kv_fraction_needed": round(r["kv_fraction_needed"], 5), "us_per_step": round(r["us_per_step"], 3)})
    x = np.array([q["kv_fraction_read"] for q in pts])
    y = np.array([q["us_per_step"] for q in pts])
    slope, icpt = np.polyfit(x, y, 1) if np.ptp(x) > 0 else (0.0, float(y.mean()))
    pred = slope * x + icpt
    ss = float(((y - y.mean()) ** 2).sum())
    r2 = 1.0 - float(((y - pred) ** 2).sum()) / ss if ss > 0 else 1.0
    return {"points": pts, "slope_us_per_unit_fraction": round(float(slope), 3), "intercept_us": round(float(icpt), 3),
            "r2": round(r2, 4)}


def summary_row(r: dict) -> dict:
    keys = ("us_per_step", "us_per_step_eager", "alg_bytes", "read_bytes", "achieved_GBps", "read_GBps",
            "kv_fraction_read", "kv_fraction_needed")
    row = {k: (round(r[k], 5) if isinstance(r[k], float) else r[k]) for k in keys}
    row["alg_frac_of_peak"] = round(r["achieved_GBps"] / PEAK_GBPS, 4)
    row["read_frac_of_peak"] = round(r["read_GBps"] / PEAK_GBPS, 4)
    return row


def kernel_name(art_mod, dev, case) -> str:
    desc = art_mod.make_desc(dev["q"], dev["k_pages"], dev["block_table"])
    return art_mod.KERNEL_NAMES[art_mod.art_decode_kernel_choice(desc, case["eps_mag"], case["eps_dir"],
                                                                 case["patience"])]


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None, help="workload name (default: the ragged long-batch decode)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration under rocprofv3)")
    ap.add_argument("--modes", default="art,full")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the other workloads, the threshold sweeps and the detector-overhead run")
    ap.add_argument("--pruned", action="store_true",
                    help="also run ART over a pruned cache (block 0 plus the newest quarter / sixteenth of the "
                         "blocks, through art_decode_visits) against full attention over the same blocks")
    ap.add_argument("--probe", action="store_true",
                    help="also run the probe-vector detector (statistics over the leading P output coordinates) "
                         "for several P: step time, detector cost and stop drift against all D coordinates")
    ap.add_argument("--importance", action="store_true",
                    help="also compare the importance-first order (key-summary pre-pass) with recency-first on the "
                         "Llama-3-8B shape and the recency control: step time, KV read, error against full attention")
    ap.add_argument("--ablation", action="store_true",
                    help="also run the detector ablation (both tests, scale only, direction only, patience 1) on "
                         "the Llama-3-8B shape with Gaussian, heavy-tailed and value-heavy K/V")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the decode has no multi-GPU path (sequences and kv-heads "
              "are independent, so a batch would split across GPUs with no communication); run with --gpus 1",
              file=sys.stderr)
        return 2

    from kv_cache_run_amd import synth, workloads

    w = workloads.BY_NAME[args.workload] if args.workload else workloads.RAGGED
    case = synth.make_case(w)
    # the CPU oracle first: its worker pool forks, which must happen before the GPU is initialised
    cpu = None
    if not args.no_cpu and "art" in args.modes.split(","):
        cpu = cpu_baseline(case)

    import torch

    from kv_cache_run_amd import art

    if not os.path.exists(art.LIB_PATH):
        from kv_cache_run_amd import build as _b

        _b.build()
    torch.cuda.set_device(0)
    dev = art.case_to_device(case)
    B = case["block_size"]
    steps_x = max(5, args.steps // 2)

    em0, ed0, p0 = case["eps_mag"], case["eps_dir"], case["patience"]
    results = {}
    for mode in [m for m in args.modes.split(",") if m]:
        if mode == "art":
            results[mode] = time_setting(case, dev, em0, ed0, p0, 0, args.steps, args.warmup)
        elif mode == "full":
            results[mode] = time_setting(case, dev, 0.0, 0.0, p0, art.ART_FLAG_FULL, args.steps, args.warmup)
        else:
            raise SystemExit(f"unknown mode {mode}")
    head_mode = "art" if "art" in results else next(iter(results))
    kname = kernel_name(art, dev, case) if head_mode == "art" else "full_split_kernel"

    extras = {}
    if not args.no_extras and "art" in results and "full" in results:
        # detector overhead: the terminating kernel with thresholds that can never pass (it folds every
        # block and runs every test) against the same kernel without the statistics, and against the
        # full-attention kernel on the same work
        keep = time_setting(case, dev, 0.0, 0.0, p0, art.ART_FLAG_KEEP_DETECTOR, steps_x, 2)
        nostats = time_setting(case, dev, 0.0, 0.0, p0, art.ART_FLAG_SKIP_STATS, steps_x, 2)
        extras["detector_overhead"] = {
            "art_kernel_all_blocks_us": round(keep["us_per_step"], 3),
            "art_kernel_all_blocks_without_statistics_us": round(nostats["us_per_step"], 3),
            "detector_cost_fraction": round(keep["us_per_step"] / nostats["us_per_step"] - 1.0, 4),
            "full_kernel_us": round(results["full"]["us_per_step"], 3),
            "ratio_to_full": round(keep["us_per_step"] / results["full"]["us_per_step"], 4),
            "note": "the terminating kernel folding every block with and without computing the statistics "
                    "(detector_cost_fraction), and against the split full-attention path (ratio_to_full)",
        }
        extras["threshold_sweep"] = {w.name: sweep(case, dev, results["art"], steps_x)}
        # every other workload, both modes; sweeps on the Llama-3-8B and 128k shapes too
        per = {w.name: {"kernel": kname, "art": summary_row(results["art"]), "full": summary_row(results["full"])}}
        del dev
        torch.cuda.empty_cache()
        for w2 in workloads.ALL:
            if w2.name == w.name:
                continue
            c2 = synth.make_case(w2)
            d2 = art.case_to_device(c2)
            ra = time_setting(c2, d2, c2["eps_mag"], c2["eps_dir"], c2["patience"], 0, steps_x, 2)
            rf = time_setting(c2, d2, 0.0, 0.0, c2["patience"], art.ART_FLAG_FULL, steps_x, 2)
            per[w2.name] = {"kernel": kernel_name(art, d2, c2), "art": summary_row(ra), "full": summary_row(rf),
                            "art_over_full": round(ra["us_per_step"] / rf["us_per_step"], 4)}
            if w2 in (workloads.LLAMA3_8B, workloads.LONG):
                extras["threshold_sweep"][w2.name] = sweep(c2, d2, ra, steps_x)
            del c2, d2
            torch.cuda.empty_cache()
        per[w.name]["art_over_full"] = round(results["art"]["us_per_step"] / results["full"]["us_per_step"], 4)
        extras["workloads"] = per
        dev = None

    if args.ablation or args.pruned or args.probe:
        dev = dev or art.case_to_device(case)
    if args.ablation:
        extras["ablation"] = ablation(steps_x, 2)
    if args.pruned:
        extras["pruned"] = pruned(case, dev, steps_x, 2)
    if args.probe:
        extras["probe"] = probe(case, dev, steps_x, 2)
    if args.importance:
        extras["importance"] = importance(steps_x, 2)

    if args.calib_copy_mib:
        src = torch.empty(args.calib_copy_mib << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()

    head = results[head_mode]
    traffic = read_traffic(kname, w.name)
    roofline = {
        "bound": "hbm",
        "kernel": kname,
        "achieved": round(head["achieved_GBps"], 1),
        "peak": PEAK_GBPS,
        "unit": "GB/s",
        "frac": round(head["achieved_GBps"] / PEAK_GBPS, 4),
        "traffic": None if traffic is None else traffic["bytes_per_launch"],
        "alg_bytes_per_launch": head["alg_bytes"],
        "read_GBps": round(head["read_GBps"], 1),
        "read_frac": round(head["read_GBps"] / PEAK_GBPS, 4),
    }
    cpu_line = None
    if cpu is not None:
        cpu_line = {"value": round(cpu["art"]["us_per_step"], 1), "unit": "us/step", "cores": cpu["art"]["cores"],
                    "kind": "oracle",
                    "sample": f"float64 NumPy oracle, ART mode, {cpu['art']['streams_timed']} of {cpu['streams']} "
                              f"streams (sequence, kv-head) with all their query heads on a pool of "
                              f"{cpu['art']['cores']} single-threaded processes (host: {cpu['host_cores']} cores, "
                              f"{cpu['cpu_model']}; at most 16 workers, the host share of one GPU), scaled to the "
                              f"whole batch",
                    "full_mode_us_per_step": round(cpu["full"]["us_per_step"], 1),
                    "one_core": {"art_us_per_step": round(cpu["art"]["one_core_us_per_step"], 1),
                                 "full_us_per_step": round(cpu["full"]["one_core_us_per_step"], 1),
                                 "art_streams_timed": cpu["art"]["one_core_streams_timed"],
                                 "full_streams_timed": cpu["full"]["one_core_streams_timed"]},
                    "detail": cpu}
    line = {
        "metric": METRIC,
        "value": round(head["us_per_step"], 3),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["us_per_step"] / 1e3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": case["kv_dtype"] + "-in/f32-accum",
        "data": "synthetic (seeded Gaussian q/K/V with planted heavy keys; no dataset or weights)",
        "config": {"workload": w.name, "mode": head_mode, "batch": case["batch"], "q_heads": case["num_q_heads"],
                   "kv_heads": case["num_kv_heads"], "head_dim": case["head_dim"],
                   "context": [int(case["seq_lens"].min()), int(case["seq_lens"].max())], "block_size": B,
                   "kv_bytes": int(case["k_pages"].nbytes + case["v_pages"].nbytes),
                   "eps_mag": case["eps_mag"], "eps_dir": case["eps_dir"], "patience": case["patience"]},
        "achieved_GBps": round(head["achieved_GBps"], 1),
        "hbm_frac": round(head["achieved_GBps"] / PEAK_GBPS, 4),
        "read_GBps": round(head["read_GBps"], 1),
        "kv_fraction_read": round(head["kv_fraction_read"], 5),
        "kv_fraction_needed": round(head["kv_fraction_needed"], 5),
        "modes": {m: {k: (round(v, 5) if isinstance(v, float) else v) for k, v in r.items()}
                  for m, r in results.items()},
        "roofline": roofline,
        "cpu_baseline": cpu_line,
        "kernel_source_hash": kernel_source_hash(),
    }
    line.update(extras)
    print(json.dumps(line))
    return 0


if __name__ == "__main__":
    sys.exit(main())
