"""ctypes binding of the C ABI in ``include/art_decode.h`` (argument marshalling only).

Every step of the decode runs in the HIP library ``libart_decode.so``; this
module only builds the descriptor from tensor shapes/dtypes, passes device
pointers and the current HIP stream, and turns status codes into exceptions.
PyTorch is used for device memory and streams.  There is no fallback: if the
library is missing the functions raise.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libart_decode.so")

ART_OK, ART_ERR_INVALID_ARG, ART_ERR_UNSUPPORTED, ART_ERR_WORKSPACE, ART_ERR_HIP = range(5)
ART_DTYPE_F32, ART_DTYPE_BF16, ART_DTYPE_FP8_E4M3FN = range(3)
ART_FLAG_NONE, ART_FLAG_FULL, ART_FLAG_KEEP_DETECTOR, ART_FLAG_SKIP_STATS = 0, 1, 2, 4
ART_FLAG_PROBE_SHIFT = 8


def art_flag_probe(p: int) -> int:
    """Flag bits of a probe-vector detector over the leading ``p`` output coordinates (p a multiple of 8)."""
    if p % 8 or not 0 <= p <= 2040:
        raise ValueError("probe size must be a multiple of 8")
    return (p // 8) << ART_FLAG_PROBE_SHIFT

EXPORTED = ("art_decode_workspace_bytes", "art_decode_workspace_init", "art_decode", "art_decode_visits",
            "art_status_string", "art_decode_version", "art_decode_kernel_choice", "art_block_key_summary",
            "art_importance_order_workspace_bytes", "art_importance_order", "art_check_inputs",
            "art_decode_reload_environment", "art_decode_noalloc", "art_decode_workspace_status")
ART_KERNEL_FULL, ART_KERNEL_SCANNERS, ART_KERNEL_LOOKBACK, ART_KERNEL_WINDOWED, ART_KERNEL_STREAM = 0, 1, 2, 3, 4
ART_KERNEL_SEGMENTS = 5
ART_CHECK_OK, ART_CHECK_SEQ_LEN, ART_CHECK_ORDER_RANGE, ART_CHECK_ORDER_REPEAT, ART_CHECK_PAGE_RANGE = 0, 1, 2, 3, 4
CHECK_NAMES = {ART_CHECK_SEQ_LEN: "sequence length outside [0, max_blocks * block_size]",
               ART_CHECK_ORDER_RANGE: "order entry outside [0, n_s)",
               ART_CHECK_ORDER_REPEAT: "order entry repeated among the visited positions",
               ART_CHECK_PAGE_RANGE: "page outside [0, num_pages)"}
KERNEL_NAMES = {ART_KERNEL_FULL: "full_split_kernel", ART_KERNEL_SCANNERS: "art_sched_kernel",
                ART_KERNEL_LOOKBACK: "art_lb_kernel", ART_KERNEL_WINDOWED: "art_win_part_kernel",
                ART_KERNEL_STREAM: "art_stream_kernel", ART_KERNEL_SEGMENTS: "art_seg_kernel"}


class ArtDecodeDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("q_dtype", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
    ]


class ArtError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


_lib = None


def _mapped_hip_runtimes() -> list:
    """Distinct HIP runtime files mapped into this process (Linux; empty where /proc is not readable)."""
    try:
        with open("/proc/self/maps") as f:
            paths = {line.split()[-1] for line in f if "libamdhip64.so" in line}
    except OSError:
        return []
    return sorted({os.path.realpath(x) for x in paths})


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m kv_cache_run_amd.build` "
                           "(there is no non-HIP fallback)")
    # torch first: it maps the HIP runtime it ships, and the library then binds to that one.  Loaded the
    # other way round, the process would hold two HIP runtimes, and pointers and streams from torch's would be
    # unknown to the library's.
    import torch  # noqa: F401

    lib = ctypes.CDLL(p)
    runtimes = _mapped_hip_runtimes()
    if len(runtimes) > 1:
        raise RuntimeError(f"two HIP runtimes are mapped ({', '.join(runtimes)}): the library must share torch's")
    vp, sz, i32, f32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_float
    lib.art_decode_workspace_bytes.argtypes = [ctypes.POINTER(ArtDecodeDesc)]
    lib.art_decode_workspace_bytes.restype = sz
    lib.art_decode_workspace_init.argtypes = [vp, sz, vp]
    lib.art_decode_workspace_init.restype = ctypes.c_int
    lib.art_decode.argtypes = [ctypes.POINTER(ArtDecodeDesc), vp, vp, vp, vp, vp, vp, vp, vp, f32, f32, i32, vp,
                               vp, vp, vp, sz, vp]
    lib.art_decode.restype = ctypes.c_int
    lib.art_decode_visits.argtypes = [ctypes.POINTER(ArtDecodeDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp, f32, f32,
                                      i32, vp, vp, vp, vp, sz, vp]
    lib.art_decode_visits.restype = ctypes.c_int
    lib.art_block_key_summary.argtypes = [ctypes.POINTER(ArtDecodeDesc), vp, vp, vp, vp, vp, vp]
    lib.art_block_key_summary.restype = ctypes.c_int
    lib.art_importance_order_workspace_bytes.argtypes = [ctypes.POINTER(ArtDecodeDesc)]
    lib.art_importance_order_workspace_bytes.restype = sz
    lib.art_importance_order.argtypes = [ctypes.POINTER(ArtDecodeDesc), vp, vp, vp, vp, vp, vp, sz, vp]
    lib.art_importance_order.restype = ctypes.c_int
    lib.art_check_inputs.argtypes = [ctypes.POINTER(ArtDecodeDesc), vp, vp, vp, vp, vp, vp]
    lib.art_check_inputs.restype = ctypes.c_int
    lib.art_status_string.argtypes = [ctypes.c_int]
    lib.art_status_string.restype = ctypes.c_char_p
    lib.art_decode_version.argtypes = []
    lib.art_decode_version.restype = i32
    lib.art_decode_kernel_choice.argtypes = [ctypes.POINTER(ArtDecodeDesc), f32, f32, i32]
    lib.art_decode_kernel_choice.restype = i32
    lib.art_decode_noalloc.argtypes = [ctypes.POINTER(ArtDecodeDesc), vp, vp, vp, vp, vp, vp, vp, vp, f32, f32, i32, vp,
                                       vp, vp, vp]
    lib.art_decode_noalloc.restype = ctypes.c_int
    lib.art_decode_workspace_status.argtypes = [vp, sz, ctypes.POINTER(i32), vp]
    lib.art_decode_workspace_status.restype = ctypes.c_int
    lib.art_decode_reload_environment.argtypes = []
    lib.art_decode_reload_environment.restype = None
    if path is None:
        _lib = lib
    return lib


def art_status_string(status: int) -> str:
    return load_library().art_status_string(int(status)).decode()


def art_decode_version() -> int:
    return int(load_library().art_decode_version())


def reload_environment() -> None:
    """Make the library re-read its tuning environment variables (it reads them once otherwise)."""
    load_library().art_decode_reload_environment()


def art_decode_kernel_choice(desc: ArtDecodeDesc, eps_mag: float, eps_dir: float, patience: int) -> int:
    """ART_KERNEL_* that art_decode would run for these arguments (raises ArtError if it would reject them)."""
    r = int(load_library().art_decode_kernel_choice(ctypes.byref(desc), float(eps_mag), float(eps_dir), int(patience)))
    if r < 0:
        _check(-r)
    return r


def _check(status: int) -> None:
    if status != ART_OK:
        raise ArtError(status, art_status_string(status))


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.float32:
        return ART_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return ART_DTYPE_BF16
    if t.dtype == torch.float8_e4m3fn:
        return ART_DTYPE_FP8_E4M3FN
    raise TypeError(f"unsupported tensor dtype {t.dtype}")


def make_desc(q, k_pages, block_table, flags: int = 0) -> ArtDecodeDesc:
    """Descriptor from q [batch, Hq, D], k_pages [pages, Hkv, B, D], block_table [batch, max_blocks]."""
    batch, hq, d = q.shape
    pages, hkv, b, d2 = k_pages.shape
    if d2 != d:
        raise ValueError("q and k_pages disagree on head_dim")
    return ArtDecodeDesc(batch, hq, hkv, d, b, block_table.shape[1], pages, _dtype_code(q), _dtype_code(k_pages),
                         flags)


def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def _stream(stream) -> Optional[int]:
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) or None


def art_decode_workspace_bytes(desc: ArtDecodeDesc) -> int:
    return int(load_library().art_decode_workspace_bytes(ctypes.byref(desc)))


def art_decode_workspace_status(workspace, stream=None) -> bool:
    """True if a bounded wait gave up in a call that used this workspace (synchronizes the stream)."""
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    failed = ctypes.c_int32(0)
    _check(load_library().art_decode_workspace_status(_ptr(workspace), nbytes, ctypes.byref(failed), _stream(stream)))
    return bool(failed.value)


def art_decode_workspace_init(workspace, stream=None) -> None:
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().art_decode_workspace_init(_ptr(workspace), nbytes, _stream(stream)))


def art_decode(q, k_pages, v_pages, block_table, block_order, seq_lens, eps_mag: float, eps_dir: float,
               patience: int, out, stop_block, *, k_scale=None, v_scale=None, blocks_fetched=None, workspace=None,
               flags: int = 0, stream=None, visit_lens=None) -> None:
    """Enqueue one ART decode step (see include/art_decode.h); tensors must be contiguous on the device.
    ``visit_lens`` (int32 [batch]) visits only the first visit_lens[s] order entries: art_decode_visits."""
    for t in (q, k_pages, v_pages, block_table, block_order, seq_lens, out, stop_block, k_scale, v_scale,
              blocks_fetched, workspace, visit_lens):
        if t is not None and not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    desc = make_desc(q, k_pages, block_table, flags)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    lib = load_library()
    if visit_lens is None:
        st = lib.art_decode(ctypes.byref(desc), _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(k_scale), _ptr(v_scale),
                            _ptr(block_table), _ptr(block_order), _ptr(seq_lens), float(eps_mag), float(eps_dir),
                            int(patience), _ptr(out), _ptr(stop_block), _ptr(blocks_fetched), _ptr(workspace), nbytes,
                            _stream(stream))
    else:
        st = lib.art_decode_visits(ctypes.byref(desc), _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(k_scale),
                                   _ptr(v_scale), _ptr(block_table), _ptr(block_order), _ptr(seq_lens),
                                   _ptr(visit_lens), float(eps_mag), float(eps_dir), int(patience), _ptr(out),
                                   _ptr(stop_block), _ptr(blocks_fetched), _ptr(workspace), nbytes,
                                   _stream(stream))
    _check(st)


def art_decode_noalloc(q, k_pages, v_pages, block_table, block_order, seq_lens, eps_mag: float, eps_dir: float,
                       patience: int, out, stop_block, *, k_scale=None, v_scale=None, blocks_fetched=None,
                       flags: int = 0, stream=None) -> None:
    """Enqueue art_decode_noalloc (no workspace: a static device scratch array, see include/art_decode.h)."""
    for t in (q, k_pages, v_pages, block_table, block_order, seq_lens, out, stop_block, k_scale, v_scale,
              blocks_fetched):
        if t is not None and not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    desc = make_desc(q, k_pages, block_table, flags)
    _check(load_library().art_decode_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(k_scale),
                                             _ptr(v_scale), _ptr(block_table), _ptr(block_order), _ptr(seq_lens),
                                             float(eps_mag), float(eps_dir), int(patience), _ptr(out),
                                             _ptr(stop_block), _ptr(blocks_fetched), _stream(stream)))


def block_key_summary(q, k_pages, block_table, seq_lens, *, k_scale=None, summary=None, stream=None):
    """Enqueue art_block_key_summary; returns the float32 [num_pages, Hkv, D] summary tensor."""
    import torch

    desc = make_desc(q, k_pages, block_table)
    if summary is None:
        summary = torch.empty((k_pages.shape[0], k_pages.shape[1], k_pages.shape[3]), dtype=torch.float32,
                              device=k_pages.device)
    _check(load_library().art_block_key_summary(ctypes.byref(desc), _ptr(k_pages), _ptr(k_scale), _ptr(block_table),
                                                _ptr(seq_lens), _ptr(summary), _stream(stream)))
    return summary


def importance_order(q, k_pages, summary, block_table, seq_lens, *, block_order=None, workspace=None, stream=None):
    """Enqueue art_importance_order; returns the int32 [batch, max_blocks] order tensor (valid below n_s).
    ``workspace``: a uint8 device tensor of art_importance_order_workspace_bytes bytes (allocated if None)."""
    import torch

    lib = load_library()
    desc = make_desc(q, k_pages, block_table)
    if block_order is None:
        block_order = torch.full(tuple(block_table.shape), -1, dtype=torch.int32, device=block_table.device)
    need = lib.art_importance_order_workspace_bytes(ctypes.byref(desc))
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=block_table.device)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.art_importance_order(ctypes.byref(desc), _ptr(q), _ptr(summary), _ptr(block_table), _ptr(seq_lens),
                                    _ptr(block_order), _ptr(workspace), nbytes, _stream(stream)))
    return block_order


def check_inputs(q, k_pages, block_table, block_order, seq_lens, *, visit_lens=None, result=None, stream=None):
    """Enqueue art_check_inputs; returns the int32 [4] device tensor (code, sequence, position, value)."""
    import torch

    desc = make_desc(q, k_pages, block_table)
    if result is None:
        result = torch.empty(4, dtype=torch.int32, device=block_table.device)
    _check(load_library().art_check_inputs(ctypes.byref(desc), _ptr(block_table), _ptr(block_order), _ptr(seq_lens),
                                           _ptr(visit_lens), _ptr(result), _stream(stream)))
    return result


def validate_inputs(q, k_pages, block_table, block_order, seq_lens, *, visit_lens=None, stream=None) -> None:
    """Run the input-contract check and wait for it; raises ValueError naming the first violation."""
    r = check_inputs(q, k_pages, block_table, block_order, seq_lens, visit_lens=visit_lens, stream=stream)
    code, s, t, val = (int(x) for x in r.cpu())
    if code != ART_CHECK_OK:
        raise ValueError(f"decode inputs: {CHECK_NAMES[code]} (sequence {s}, visit position {t}, value {val})")


class Decoder:
    """Holds a device workspace for one descriptor shape and calls :func:`art_decode`.

    With ``check_inputs`` (default: environment ART_CHECK_INPUTS=1) every call first runs the input-contract
    check and waits for it (a debugging aid: it synchronizes the stream)."""

    def __init__(self, q, k_pages, block_table, device=None, check_inputs=None):
        import torch

        self.check = os.environ.get("ART_CHECK_INPUTS") == "1" if check_inputs is None else bool(check_inputs)
        self.desc = make_desc(q, k_pages, block_table)
        nbytes = art_decode_workspace_bytes(self.desc)
        self.workspace = None
        if nbytes:
            self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=device or q.device)
            art_decode_workspace_init(self.workspace)

    def __call__(self, q, k_pages, v_pages, block_table, block_order, seq_lens, eps_mag, eps_dir, patience, *,
                 k_scale=None, v_scale=None, out=None, stop_block=None, blocks_fetched=None, flags=0, stream=None,
                 visit_lens=None):
        import torch

        batch, hq, d = q.shape
        if self.check:
            validate_inputs(q, k_pages, block_table, block_order, seq_lens, visit_lens=visit_lens, stream=stream)
        if out is None:
            out = torch.empty((batch, hq, d), dtype=torch.float32, device=q.device)
        if stop_block is None:
            stop_block = torch.empty((batch, hq), dtype=torch.int32, device=q.device)
        art_decode(q, k_pages, v_pages, block_table, block_order, seq_lens, eps_mag, eps_dir, patience, out,
                   stop_block, k_scale=k_scale, v_scale=v_scale, blocks_fetched=blocks_fetched,
                   workspace=self.workspace, flags=flags, stream=stream, visit_lens=visit_lens)
        return out, stop_block


def case_to_device(case: dict, device="cuda") -> dict:
    """Copy a generated case (host NumPy storage arrays) to device tensors of the matching dtypes."""
    import numpy as np
    import torch

    def kv(a, dtype):
        if dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
        if dtype == "fp8_e4m3fn":
            return torch.from_numpy(np.ascontiguousarray(a)).to(device).view(torch.float8_e4m3fn)
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)

    d = {
        "q": kv(case["q"], case["q_dtype"]),
        "k_pages": kv(case["k_pages"], case["kv_dtype"]),
        "v_pages": kv(case["v_pages"], case["kv_dtype"]),
        "block_table": torch.from_numpy(case["block_table"]).to(device),
        "block_order": torch.from_numpy(case["block_order"]).to(device),
        "seq_lens": torch.from_numpy(case["seq_lens"]).to(device),
        "k_scale": None if case.get("k_scale") is None else torch.from_numpy(case["k_scale"]).to(device),
        "v_scale": None if case.get("v_scale") is None else torch.from_numpy(case["v_scale"]).to(device),
    }
    return d
