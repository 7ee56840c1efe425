"""The synthetic decode workloads: shapes, storage types, planted-key recipe, ART thresholds.

Each workload is one decode step of one attention layer over a paged KV cache.
The shapes stand in for the models the ART explainer evaluates on (its
Technical Summary section 4 names Mistral-7B-Instruct and Llama-3.1-70B on
LongBench); neither the dataset nor trained weights are available, so the
attention structure is synthetic: Gaussian q/K/V with a planted set of heavy
keys aligned with the query group, which makes the attention heavy-tailed.
"""

from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Tuple, Union


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    q_dtype: str            # "f32" | "bf16"
    kv_dtype: str           # "f32" | "bf16" | "fp8_e4m3fn"
    context: Union[int, Tuple[int, int]]   # fixed length, or (lo, hi) drawn per sequence
    heavy: tuple            # ("frac", f) | ("frac_range", lo, hi) | ("spans", count, length)
    eps_mag: float
    eps_dir: float
    patience: int
    seed: int
    order: str = "sink_then_newest"        # block 0 first, then newest to oldest
    tail_fill: bool = True                 # poison rows past seq_len in the last page
    kv_dist: str = "normal"                # K/V entries: "normal" N(0, 1) | "student_t3" (3 degrees of freedom)
    value_heavy: tuple = ()                # () | (f, gain): round(f * L) positions in the oldest quarter, V *= gain

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


TINY = Workload(
    name="tiny-f32-b1-h1-d64-ctx1024-blk16", batch=1, num_q_heads=1, num_kv_heads=1, head_dim=64,
    block_size=16, q_dtype="f32", kv_dtype="f32", context=1024, heavy=("frac", 0.05),
    eps_mag=1e-3, eps_dir=1e-4, patience=3, seed=1)

LLAMA3_8B = Workload(
    name="llama3-8b-gqa4-bf16-b8-ctx8192-blk16", batch=8, num_q_heads=32, num_kv_heads=8, head_dim=128,
    block_size=16, q_dtype="bf16", kv_dtype="bf16", context=8192, heavy=("frac", 0.03),
    eps_mag=1e-3, eps_dir=1e-4, patience=4, seed=2)

RAGGED = Workload(
    name="ragged-gqa4-bf16-b32-ctx4k-32k-blk16", batch=32, num_q_heads=32, num_kv_heads=8, head_dim=128,
    block_size=16, q_dtype="bf16", kv_dtype="bf16", context=(4096, 32768), heavy=("frac_range", 0.005, 0.10),
    eps_mag=1e-3, eps_dir=1e-4, patience=4, seed=3)

LONG = Workload(
    name="long-gqa8-bf16-b4-ctx131072-blk32", batch=4, num_q_heads=64, num_kv_heads=8, head_dim=128,
    block_size=32, q_dtype="bf16", kv_dtype="bf16", context=131072, heavy=("spans", 20, 64),
    eps_mag=5e-4, eps_dir=5e-5, patience=6, seed=4)

QWEN_FP8 = Workload(
    name="qwen2.5-7b-gqa7-fp8kv-b64-ctx16384-blk16", batch=64, num_q_heads=28, num_kv_heads=4, head_dim=128,
    block_size=16, q_dtype="bf16", kv_dtype="fp8_e4m3fn", context=16384, heavy=("frac", 0.03),
    eps_mag=1e-3, eps_dir=1e-4, patience=4, seed=5)

ALL = (TINY, LLAMA3_8B, RAGGED, LONG, QWEN_FP8)

# Inputs for the ablation of the detector (scale-only, direction-only,
# patience 1), all on the Llama-3-8B shape: heavy-tailed K/V; a few
# value-heavy tokens (ordinary keys, values 32x larger) among the oldest,
# which the default order visits last -- a head can look converged before it
# has seen what matters; and, as the control, heavy keys only among the
# newest 5% of tokens, which the default order visits first.
HEAVY_TAIL = LLAMA3_8B.scaled(name="heavytail-t3-gqa4-bf16-b8-ctx8192-blk16", kv_dist="student_t3", seed=6)
VALUE_HEAVY = LLAMA3_8B.scaled(name="valueheavy-gqa4-bf16-b8-ctx8192-blk16", value_heavy=(0.002, 32.0), seed=7)
RECENT = LLAMA3_8B.scaled(name="recent-gqa4-bf16-b8-ctx8192-blk16", heavy=("recent", 0.01, 0.05), seed=8)
ABLATION = (LLAMA3_8B, HEAVY_TAIL, VALUE_HEAVY, RECENT)

BY_NAME = {w.name: w for w in ALL + ABLATION}
