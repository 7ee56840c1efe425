"""The C-ABI library: exports, host-side validation (no GPU needed, no device call made)."""

import ctypes
import os
import re

import pytest

from kv_cache_run_amd import art

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(art.LIB_PATH):
        from kv_cache_run_amd import build

        build.build()
    return art.load_library()


def _declared_functions():
    names = []
    inc = os.path.join(ROOT, "include")
    for fn in sorted(os.listdir(inc)):
        if fn.endswith(".h"):
            text = open(os.path.join(inc, fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"\b(art_[a-z0-9_]+)\s*\(", text)
    return sorted(set(names))


def test_every_declared_function_is_exported(lib):
    names = _declared_functions()
    assert "art_decode" in names and len(names) >= 5
    for n in names:
        assert hasattr(lib, n), n
    assert set(art.EXPORTED) == set(names)


def test_status_strings_and_version(lib):
    for s in range(5):
        assert art.art_status_string(s).startswith("ART_")
    assert "unknown" in art.art_status_string(99)
    assert art.art_decode_version() >= 100


def _desc(**kw):
    base = dict(batch=2, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16, max_blocks_per_seq=64,
                num_pages=128, q_dtype=art.ART_DTYPE_BF16, kv_dtype=art.ART_DTYPE_BF16, flags=0)
    base.update(kw)
    return art.ArtDecodeDesc(**base)


FAKE = 0x10000  # aligned, never dereferenced: every case below fails validation first


def _call(lib, desc, *, q=FAKE, k=FAKE, v=FAKE, ks=None, vs=None, bt=FAKE, bo=FAKE, sl=FAKE, em=1e-3, ed=1e-4, p=4,
          out=FAKE, stop=FAKE, fetched=None, ws=FAKE, wsb=1 << 30):
    return lib.art_decode(ctypes.byref(desc) if desc is not None else None, q, k, v, ks, vs, bt, bo, sl, em, ed, p,
                          out, stop, fetched, ws, wsb, None)


def test_validation_errors_return_before_any_device_call(lib):
    E_ARG, E_UNS, E_WS = art.ART_ERR_INVALID_ARG, art.ART_ERR_UNSUPPORTED, art.ART_ERR_WORKSPACE
    assert _call(lib, None) == E_ARG
    assert _call(lib, _desc(num_q_heads=30)) == E_ARG                    # Hq % Hkv
    assert _call(lib, _desc(num_q_heads=136, num_kv_heads=8)) == E_UNS   # g = 17
    assert _call(lib, _desc(head_dim=96)) == E_UNS
    assert _call(lib, _desc(block_size=8)) == E_UNS
    assert _call(lib, _desc(q_dtype=art.ART_DTYPE_F32)) == E_UNS          # f32 q with bf16 KV
    assert _call(lib, _desc(kv_dtype=7)) == E_ARG
    assert _call(lib, _desc(batch=-1)) == E_ARG
    assert _call(lib, _desc(flags=8)) == E_ARG
    assert _call(lib, _desc(), em=float("nan")) == E_ARG
    assert _call(lib, _desc(), ed=-1e-4) == E_ARG
    assert _call(lib, _desc(), p=0) == E_ARG
    assert _call(lib, _desc(), q=None) == E_ARG
    assert _call(lib, _desc(), stop=None) == E_ARG
    assert _call(lib, _desc(), k=FAKE + 8) == E_ARG                        # 16-byte alignment
    assert _call(lib, _desc(), ks=FAKE) == E_ARG                           # scales only for fp8
    assert _call(lib, _desc(kv_dtype=art.ART_DTYPE_FP8_E4M3FN)) == E_ARG   # fp8 needs scales
    assert _call(lib, _desc(), ws=None) == E_WS
    assert _call(lib, _desc(), wsb=16) == E_WS
    assert _call(lib, _desc(), ws=FAKE + 64) == E_ARG                      # 256-byte alignment
    # an empty batch is valid and enqueues nothing
    assert _call(lib, _desc(batch=0), ws=None, wsb=0) == art.ART_OK


def test_workspace_size_query(lib):
    assert art.art_decode_workspace_bytes(_desc(head_dim=96)) == 0
    n = art.art_decode_workspace_bytes(_desc())
    assert n > 0 and n % 256 == 0
    assert art.art_decode_workspace_bytes(_desc(batch=0)) == 0
    assert lib.art_decode_workspace_init(None, 0, None) == art.ART_OK
    assert lib.art_decode_workspace_init(None, 256, None) == art.ART_ERR_INVALID_ARG


@pytest.fixture()
def env(monkeypatch):
    """Set or clear tuning variables; the library reads them again after each change and once more at the end."""
    class Env:
        def set(self, k, v):
            monkeypatch.setenv(k, v)
            art.reload_environment()

        def unset(self, k):
            monkeypatch.delenv(k, raising=False)
            art.reload_environment()
    yield Env()
    monkeypatch.undo()
    art.reload_environment()


def test_kernel_choice_follows_the_knob_and_the_mode(lib, env):
    """Which kernel a call would run, without any device call: forced schedulers, full mode, rejected args."""
    long_desc = _desc(batch=4, num_q_heads=64, num_kv_heads=8, block_size=32, max_blocks_per_seq=4096)
    qwen_desc = _desc(batch=64, num_q_heads=28, num_kv_heads=4, max_blocks_per_seq=1024,
                      kv_dtype=art.ART_DTYPE_FP8_E4M3FN)
    # auto (no device here: 256 CUs assumed), groups of up to 8 heads: segments for few long streams and for
    # groups of more than 4 heads with long streams, else the stream kernel; larger groups: windows for few
    # long streams, look-back for long streams, else scanners
    env.unset("ART_SCHED")
    assert art.art_decode_kernel_choice(long_desc, 5e-4, 5e-5, 6) == art.ART_KERNEL_SEGMENTS
    assert art.art_decode_kernel_choice(qwen_desc, 1e-3, 1e-4, 4) == art.ART_KERNEL_SEGMENTS
    assert art.art_decode_kernel_choice(_desc(num_q_heads=56, max_blocks_per_seq=64), 1e-3, 1e-4, 4) == \
        art.ART_KERNEL_STREAM
    assert art.art_decode_kernel_choice(_desc(), 1e-3, 1e-4, 4) == art.ART_KERNEL_STREAM
    assert art.art_decode_kernel_choice(_desc(num_q_heads=128, max_blocks_per_seq=256), 1e-3, 1e-4, 4) == \
        art.ART_KERNEL_LOOKBACK
    assert art.art_decode_kernel_choice(_desc(num_q_heads=128, max_blocks_per_seq=16), 1e-3, 1e-4, 4) == \
        art.ART_KERNEL_SCANNERS
    assert art.art_decode_kernel_choice(_desc(max_blocks_per_seq=8192), 1e-3, 1e-4, 4) == art.ART_KERNEL_SEGMENTS
    assert art.art_decode_kernel_choice(_desc(num_q_heads=128, max_blocks_per_seq=8192), 1e-3, 1e-4, 4) == \
        art.ART_KERNEL_WINDOWED
    env.set("ART_SCHED", "seg")
    assert art.art_decode_kernel_choice(_desc(), 1e-3, 1e-4, 4) == art.ART_KERNEL_SEGMENTS
    # groups of more than 8 heads, or pass counts past what its status words hold: scanners
    assert art.art_decode_kernel_choice(_desc(num_q_heads=128), 1e-3, 1e-4, 4) == art.ART_KERNEL_SCANNERS
    assert art.art_decode_kernel_choice(_desc(), 1e-3, 1e-4, 1 << 26) == art.ART_KERNEL_SCANNERS
    env.set("ART_SCHED", "stream")
    assert art.art_decode_kernel_choice(long_desc, 1e-3, 1e-4, 4) == art.ART_KERNEL_STREAM
    # groups of more than 8 heads: the stream kernel takes none, scanners instead
    assert art.art_decode_kernel_choice(_desc(num_q_heads=128), 1e-3, 1e-4, 4) == art.ART_KERNEL_SCANNERS
    env.set("ART_SCHED", "scan")
    assert art.art_decode_kernel_choice(long_desc, 1e-3, 1e-4, 4) == art.ART_KERNEL_SCANNERS
    env.set("ART_SCHED", "win")
    assert art.art_decode_kernel_choice(_desc(), 1e-3, 1e-4, 4) == art.ART_KERNEL_WINDOWED
    # the windowed path carries the pass count as a float: beyond 2^24, scanners
    assert art.art_decode_kernel_choice(_desc(), 1e-3, 1e-4, (1 << 24) + 1) == art.ART_KERNEL_SCANNERS
    env.set("ART_SCHED", "lb")
    assert art.art_decode_kernel_choice(_desc(), 1e-3, 1e-4, 4) == art.ART_KERNEL_LOOKBACK
    # the environment is read once: a change without the reload call has no effect
    os.environ["ART_SCHED"] = "scan"
    assert art.art_decode_kernel_choice(_desc(), 1e-3, 1e-4, 4) == art.ART_KERNEL_LOOKBACK
    env.set("ART_SCHED", "lb")
    # pass counts above 2047 do not fit the look-back records: scanners
    assert art.art_decode_kernel_choice(_desc(), 1e-3, 1e-4, 2048) == art.ART_KERNEL_SCANNERS
    # full attention: the flag, or a zero threshold without ART_FLAG_KEEP_DETECTOR
    assert art.art_decode_kernel_choice(_desc(flags=art.ART_FLAG_FULL), 1e-3, 1e-4, 4) == art.ART_KERNEL_FULL
    assert art.art_decode_kernel_choice(_desc(), 0.0, 1e-4, 4) == art.ART_KERNEL_FULL
    assert art.art_decode_kernel_choice(_desc(flags=art.ART_FLAG_KEEP_DETECTOR), 0.0, 1e-4, 4) == art.ART_KERNEL_LOOKBACK
    # the measurement flag runs the terminating kernel too, whatever the thresholds
    assert art.art_decode_kernel_choice(_desc(flags=art.ART_FLAG_SKIP_STATS), 0.0, 0.0, 4) == art.ART_KERNEL_LOOKBACK
    assert art.art_decode_kernel_choice(_desc(flags=art.ART_FLAG_SKIP_STATS), 1e-3, 1e-4, 4) == art.ART_KERNEL_LOOKBACK
    with pytest.raises(art.ArtError):   # an unknown flag bit
        art.art_decode_kernel_choice(_desc(flags=8), 1e-3, 1e-4, 4)
    for bad in [dict(p=0), dict(em=-1.0), dict(ed=float("nan"))]:
        with pytest.raises(art.ArtError):
            art.art_decode_kernel_choice(_desc(), bad.get("em", 1e-3), bad.get("ed", 1e-4), bad.get("p", 4))
    with pytest.raises(art.ArtError):
        art.art_decode_kernel_choice(_desc(head_dim=96), 1e-3, 1e-4, 4)


def test_visits_entry_point_validates_like_art_decode(lib):
    """art_decode_visits: NULL visit_lens is art_decode; a misaligned visit_lens is rejected before any work."""
    args = lambda vl: (ctypes.byref(_desc()), FAKE, FAKE, FAKE, None, None, FAKE, FAKE, FAKE, vl, 1e-3, 1e-4, 4,
                       FAKE, FAKE, None, FAKE, 16, None)
    assert lib.art_decode_visits(*args(None)) == art.ART_ERR_WORKSPACE      # same checks, same order
    assert lib.art_decode_visits(*args(FAKE + 2)) == art.ART_ERR_INVALID_ARG  # 4-byte alignment


def test_probe_flag_is_validated(lib):
    """Probe sizes up to D are accepted (the call then fails only on the fake workspace); beyond D, rejected."""
    ok = _desc(flags=art.art_flag_probe(64))
    assert art.art_decode_workspace_bytes(ok) > 0
    assert art.art_decode_workspace_bytes(_desc(flags=art.art_flag_probe(128))) > 0
    assert art.art_decode_workspace_bytes(_desc(flags=art.art_flag_probe(136))) == 0   # P > D
    assert _call(lib, _desc(flags=art.art_flag_probe(136))) == art.ART_ERR_INVALID_ARG
    assert _call(lib, _desc(flags=art.art_flag_probe(8)), wsb=16) == art.ART_ERR_WORKSPACE


def test_importance_order_entry_points_validate(lib):
    """Workspace size query and the checks art_importance_order makes before any work."""
    d = _desc()
    need = lib.art_importance_order_workspace_bytes(ctypes.byref(d))
    assert need >= 2 * 64 * 4 and need % 256 == 0
    call = lambda desc, ws, wsb: lib.art_importance_order(ctypes.byref(desc), FAKE, FAKE, FAKE, FAKE, FAKE, ws, wsb,
                                                          None)
    assert call(d, FAKE, 16) == art.ART_ERR_WORKSPACE
    assert call(d, FAKE + 64, need) == art.ART_ERR_INVALID_ARG                    # 256-byte alignment
    assert call(_desc(max_blocks_per_seq=4097), FAKE, 1 << 30) == art.ART_ERR_UNSUPPORTED
    assert lib.art_importance_order(ctypes.byref(d), FAKE, FAKE + 4, FAKE, FAKE, FAKE, FAKE, need,
                                    None) == art.ART_ERR_INVALID_ARG             # summary: 16-byte alignment
    assert lib.art_block_key_summary(ctypes.byref(d), FAKE, None, FAKE, FAKE, None, None) == art.ART_ERR_INVALID_ARG


def test_check_inputs_entry_point_validates(lib):
    """art_check_inputs rejects NULL and misaligned pointers, a bad descriptor and too-long rows before any work."""
    d = _desc()
    call = lambda desc, bt, bo, sl, vl, res: lib.art_check_inputs(ctypes.byref(desc), bt, bo, sl, vl, res, None)
    assert call(d, None, FAKE, FAKE, None, FAKE) == art.ART_ERR_INVALID_ARG
    assert call(d, FAKE, FAKE, FAKE, None, None) == art.ART_ERR_INVALID_ARG
    assert call(d, FAKE, FAKE, FAKE, None, FAKE + 4) == art.ART_ERR_INVALID_ARG   # result: 8-byte alignment
    assert call(d, FAKE + 2, FAKE, FAKE, None, FAKE) == art.ART_ERR_INVALID_ARG   # tables: 4-byte alignment
    assert call(d, FAKE, FAKE, FAKE, FAKE + 1, FAKE) == art.ART_ERR_INVALID_ARG
    assert call(_desc(max_blocks_per_seq=(1 << 18) + 1), FAKE, FAKE, FAKE, None, FAKE) == art.ART_ERR_UNSUPPORTED
    assert call(_desc(num_kv_heads=3), FAKE, FAKE, FAKE, None, FAKE) != art.ART_OK


def test_noalloc_rejects_partials_past_the_static_scratch(lib):
    """art_decode_noalloc: full attention whose piece partials would pass the 8 MiB static array is refused
    before any device call (128 sequences x 8 kv-heads of 16 query heads with 256 workgroups: (1024 + 256)
    pieces x 16 x 130 floats = 10.6 MB, past 8 MiB less the 64 KiB of counters); the same descriptor in ART
    mode needs no scratch but the call then reaches the device, which this host test does not do."""
    d = _desc(batch=128, num_q_heads=128, num_kv_heads=8, max_blocks_per_seq=64, num_pages=65536)
    args = lambda em: (ctypes.byref(d), FAKE, FAKE, FAKE, None, None, FAKE, FAKE, FAKE, em, em, 1, FAKE, FAKE, None,
                       None)
    assert lib.art_decode_noalloc(*args(0.0)) == art.ART_ERR_WORKSPACE
    # argument checks come first, as in art_decode
    assert lib.art_decode_noalloc(ctypes.byref(d), None, FAKE, FAKE, None, None, FAKE, FAKE, FAKE, 0.0, 0.0, 1,
                                  FAKE, FAKE, None, None) == art.ART_ERR_INVALID_ARG


def test_library_shares_torchs_hip_runtime():
    """Loading the library (which imports torch first) leaves exactly one HIP runtime mapped, whatever was
    imported before."""
    import subprocess
    import sys

    code = ("from kv_cache_run_amd import art; art.load_library(); "
            "import torch; print(len(art._mapped_hip_runtimes()))")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip().splitlines()[-1] == "1"
