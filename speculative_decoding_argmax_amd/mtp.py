"""Python binding of the MTP draft / verify C ABI (``include/mtp.h``).

Argument marshalling only: tensors are passed as device pointers taken from
``data_ptr()``, the stream is torch's current HIP stream, and every step of the
path runs in the library's kernels. The library is loaded from
``speculative_decoding_argmax_amd/lib/libmtp.so`` (build it with
``python -m speculative_decoding_argmax_amd.build``); importing this module
raises if it is missing.

Function names match the C entry points. bfloat16 tensors may be passed as
``torch.bfloat16`` or as ``torch.int16`` / ``torch.uint16`` bit patterns.
"""

from __future__ import annotations

import ctypes
import os
import re
from typing import List, Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libmtp.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "mtp.h")

MTP_OK = 0
MTP_ERR_INVALID_ARG = 1
MTP_ERR_UNSUPPORTED = 2
MTP_ERR_WORKSPACE = 3
MTP_ERR_IDS = 4
MTP_ERR_HIP = 5

MTP_PATH_AUTO = 0
MTP_PATH_VALU = 1
MTP_PATH_MFMA = 2

MTP_MAX_K = 15
MTP_MAX_ROWS = 4096
MTP_NOALLOC_MAX_ROWS = 1024
MTP_MAX_HIDDEN = 16384


class MTPError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)}"
                         + (f" (hipError {last_hip_error()})" if status == MTP_ERR_HIP else ""))


class mtp_config(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int), ("blocks_per_cu", ctypes.c_int),
                ("reserved", ctypes.c_int * 6)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"HIP library not built: {LIB_PATH} is missing "
            "(run python -m speculative_decoding_argmax_amd.build)")
    # One HIP runtime per process: torch ships its own libamdhip64.so.7. If
    # the library were loaded first, the dynamic linker would bind it to the
    # system copy, torch would then bring in a second runtime, and the
    # library's launches would find no device. Importing torch first makes
    # the library bind to the runtime that owns torch's memory and streams.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    I = ctypes.c_int
    I64 = ctypes.c_int64
    S = ctypes.c_size_t
    sig = {
        "mtp_status_string": ([I], ctypes.c_char_p),
        "mtp_last_hip_error": ([], I),
        "mtp_time_next_call": ([P, P], None),
        "mtp_version": ([], I),
        "mtp_validate_ids": ([P, I64, I64], I),
        "mtp_draft_workspace_bytes": ([I, I64, I], S),
        "mtp_verify_workspace_bytes": ([I, I, I64, I], S),
        "mtp_workspace_init": ([P, S, P], I),
        "mtp_pack_candidates": ([P, I64, I, P, I64, P, P], I),
        "mtp_draft_argmax": ([P, I, I, P, P, I64, P, P, P, S, P], I),
        "mtp_draft_argmax_cfg": ([P, I, I, P, P, I64, P, P, P, S, P, P], I),
        "mtp_verify_accept": ([P, I, I, I, P, I64, P, P, P, P, P, P, S, P], I),
        "mtp_verify_accept_cfg": ([P, I, I, I, P, I64, P, P, P, P, P, P, S, P, P], I),
        "mtp_verify_accept_noalloc": ([P, I, I, I, P, I64, P, P, P, P, P, P], I),
        "mtp_tiled_bytes": ([I64, I], S),
        "mtp_pack_tiled": ([P, I64, I, P, I64, P, S, P], I),
        "mtp_draft_argmax_tiled": ([P, I, I, P, P, I64, P, P, P, S, P], I),
        "mtp_draft_argmax_tiled_cfg": ([P, I, I, P, P, I64, P, P, P, S, P, P], I),
        "mtp_verify_accept_tiled": ([P, I, I, I, P, I64, P, P, P, P, P, P, S, P], I),
        "mtp_verify_accept_tiled_cfg": ([P, I, I, I, P, I64, P, P, P, P, P, P, S, P, P], I),
        "mtp_draft_argmax_gather": ([P, I, I, P, I64, P, I64, P, P, P, S, P], I),
        "mtp_draft_argmax_gather_cfg": ([P, I, I, P, I64, P, I64, P, P, P, S, P, P], I),
        "mtp_fp8_table_bytes": ([I64, I], S),
        "mtp_mxfp4_table_bytes": ([I64, I], S),
        "mtp_mxfp4_scale_bytes": ([I64, I], S),
        "mtp_pack_candidates_mxfp4": ([P, I64, I, P, I64, P, P, P], I),
        "mtp_pack_candidates_mxfp4_rule": ([P, I64, I, P, I64, P, P, I, P], I),
        "mtp_draft_argmax_mxfp4": ([P, I, I, P, P, P, I64, P, P, P, S, P], I),
        "mtp_draft_argmax_mxfp4_cfg": ([P, I, I, P, P, P, I64, P, P, P, S, P, P], I),
        "mtp_draft_argmax_mxfp4_gather": ([P, I, I, P, P, I64, P, I64, P, P, P, S, P], I),
        "mtp_draft_argmax_mxfp4_gather_cfg": ([P, I, I, P, P, I64, P, I64, P, P, P, S, P, P],
                                              I),
        "mtp_pack_candidates_fp8": ([P, I64, I, P, I64, P, P, P], I),
        "mtp_draft_argmax_fp8": ([P, I, I, P, P, P, I64, P, P, P, S, P], I),
        "mtp_draft_argmax_fp8_cfg": ([P, I, I, P, P, P, I64, P, P, P, S, P, P], I),
        "mtp_draft_argmax_fp8_gather": ([P, I, I, P, P, I64, P, I64, P, P, P, S, P], I),
        "mtp_draft_argmax_fp8_gather_cfg": ([P, I, I, P, P, I64, P, I64, P, P, P, S, P, P],
                                            I),
        "mtp_tiled_fp8_bytes": ([I64, I], S),
        "mtp_tiled_mxfp4_bytes": ([I64, I], S),
        "mtp_tiled_mxfp4_scale_bytes": ([I64, I], S),
        "mtp_pack_tiled_mxfp4": ([P, I64, I, P, I64, P, S, P, S, P], I),
        "mtp_pack_tiled_mxfp4_rule": ([P, I64, I, P, I64, P, S, P, S, I, P], I),
        "mtp_draft_argmax_tiled_mxfp4": ([P, I, I, P, P, P, I64, P, P, P, S, P], I),
        "mtp_draft_argmax_tiled_mxfp4_cfg": ([P, I, I, P, P, P, I64, P, P, P, S, P, P], I),
        "mtp_pack_tiled_fp8": ([P, I64, I, P, I64, P, S, P, P], I),
        "mtp_draft_argmax_tiled_fp8": ([P, I, I, P, P, P, I64, P, P, P, S, P], I),
        "mtp_draft_argmax_tiled_fp8_cfg": ([P, I, I, P, P, P, I64, P, P, P, S, P, P], I),
        "mtp_stream_read": ([P, S, P, P], I),
        "mtp_probe_atomic": ([P, I, I, I, P, P], I),
        "mtp_graph_begin": ([P], I),
        "mtp_graph_end": ([P, ctypes.POINTER(P)], I),
        "mtp_graph_launch": ([P, P], I),
        "mtp_graph_destroy": ([P], None),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    # the HIP runtime the library is bound to (torch's): event timing of the
    # calls timed with mtp_time_next_call, whose events torch did not record
    lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), P, P]
    lib.hipEventElapsedTime.restype = I
    return lib


lib = _load()


def header_symbols(path: str = HEADER) -> List[str]:
    """Entry points declared in include/mtp.h."""
    text = open(path).read()
    return sorted(set(re.findall(r"\b(mtp_[a-z0-9_]+)\s*\(", text)))


def status_string(status: int) -> str:
    return lib.mtp_status_string(int(status)).decode()


def last_hip_error() -> int:
    return int(lib.mtp_last_hip_error())


def timing_events(n: int, stream=None):
    """n torch.cuda.Event(enable_timing=True) events backed by HIP events
    (torch creates the HIP event on an event's first record, so each is
    recorded once here, then the stream is synchronised): the events that
    mtp_time_next_call takes. Create them outside any timed region."""
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in evs:
        e.record(s)
    s.synchronize()
    return evs


def mtp_time_next_call(start=None, stop=None) -> None:
    """Time the next draft / verify call of this thread between two events of
    timing_events() (a measurement aid; see include/mtp.h): the events take
    the call's own kernel start and end; read them with elapsed_ms()."""
    def handle(ev):
        if ev is None:
            return None
        if not ev.cuda_event:
            raise ValueError("event has no HIP event yet: create it with timing_events()")
        return ctypes.c_void_p(ev.cuda_event)
    lib.mtp_time_next_call(handle(start), handle(stop))


def elapsed_ms(start, stop) -> float:
    """Milliseconds between two events stamped by a call timed with
    mtp_time_next_call (hipEventElapsedTime; torch's own elapsed_time only
    accepts events that torch recorded)."""
    ms = ctypes.c_float(0.0)
    rc = lib.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(start.cuda_event),
                                 ctypes.c_void_p(stop.cuda_event))
    if rc != 0:
        raise RuntimeError(f"hipEventElapsedTime failed (hipError {rc})")
    return float(ms.value)


def _check(status: int, what: str) -> None:
    if status != MTP_OK:
        raise MTPError(status, what)


# --- tensor marshalling ---------------------------------------------------------

def _torch():
    import torch
    return torch


def _ptr(t, what: str, dtypes, device: bool = True, allow_none: bool = False):
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{what} is required")
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{what}: dtype {t.dtype} not in {dtypes}")
    if device and not t.is_cuda:
        raise ValueError(f"{what} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _bf16_types():
    torch = _torch()
    out = [torch.bfloat16, torch.int16]
    if hasattr(torch, "uint16"):
        out.append(torch.uint16)
    return tuple(out)


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _cfg(path: int = MTP_PATH_AUTO, blocks_per_cu: int = 0):
    c = mtp_config()
    c.path = path
    c.blocks_per_cu = blocks_per_cu
    return c


# --- entry points ---------------------------------------------------------------

def mtp_validate_ids(ids_host, V: int) -> int:
    """Host check of candidate ids (numpy int32 array or CPU tensor). Returns the status."""
    import numpy as np
    a = np.ascontiguousarray(np.asarray(ids_host), dtype=np.int32)
    return int(lib.mtp_validate_ids(a.ctypes.data_as(ctypes.c_void_p), a.size, int(V)))


def mtp_draft_workspace_bytes(M: int, C: int, H: int) -> int:
    return int(lib.mtp_draft_workspace_bytes(M, C, H))


def mtp_verify_workspace_bytes(B: int, k: int, V: int, H: int) -> int:
    return int(lib.mtp_verify_workspace_bytes(B, k, V, H))


def alloc_workspace(nbytes: int, device=None, stream=None):
    """Allocate (torch) and zero (mtp_workspace_init) a workspace of nbytes.

    With ``stream`` given, the block is allocated on that stream: torch's
    caching allocator then hands it out again only to later work on the same
    stream, so a workspace that the caller drops right after an asynchronous
    call on a side stream is never reused while that call still runs.
    """
    torch = _torch()
    n = max(8, (int(nbytes) + 7) // 8 * 8)
    if stream is None:
        ws = torch.empty(n // 8, dtype=torch.int64, device=device or "cuda")
    else:
        with torch.cuda.stream(stream):
            ws = torch.empty(n // 8, dtype=torch.int64, device=device or "cuda")
    mtp_workspace_init(ws, stream=stream)
    return ws


_capturing = 0


def _no_alloc_in_capture(what: str) -> None:
    if _capturing:
        raise ValueError(f"{what}: pass ws explicitly; a call captured into a graph "
                         "must not allocate (the graph keeps the workspace pointer)")


def mtp_workspace_init(ws, stream=None) -> None:
    torch = _torch()
    p = _ptr(ws, "ws", (torch.int64, torch.uint8, torch.int32))
    _check(lib.mtp_workspace_init(p, ws.numel() * ws.element_size(), _stream(stream)),
           "mtp_workspace_init")


def mtp_pack_candidates(head, ids, table, stream=None) -> None:
    torch = _torch()
    V, H = head.shape
    C = ids.numel()
    if tuple(table.shape) != (C, H):
        raise ValueError("table must be [C][H]")
    _check(lib.mtp_pack_candidates(_ptr(head, "head", _bf16_types()), V, H,
                                   _ptr(ids, "ids", (torch.int32,)), C,
                                   _ptr(table, "table", _bf16_types()), _stream(stream)),
           "mtp_pack_candidates")


def mtp_draft_argmax(hidden, table, ids, out_ids, out_logit=None, ws=None, stream=None,
                     path: int = MTP_PATH_AUTO, blocks_per_cu: int = 0) -> None:
    """Draft GEMV + argmax: out_ids[m] = ids[argmax_i hidden[m] . table[i]]."""
    torch = _torch()
    M, H = hidden.shape
    C, H2 = table.shape
    if H != H2:
        raise ValueError("hidden and table widths differ")
    if ids is not None and ids.numel() != C:
        raise ValueError("ids must have C entries")
    if out_ids.numel() != M or (out_logit is not None and out_logit.numel() != M):
        raise ValueError("outputs must have M entries")
    if ws is None:
        _no_alloc_in_capture("mtp_draft_argmax")
        ws = alloc_workspace(mtp_draft_workspace_bytes(M, C, H), hidden.device, stream)
    cfg = _cfg(path, blocks_per_cu)
    _check(lib.mtp_draft_argmax_cfg(
        _ptr(hidden, "hidden", _bf16_types()), M, H, _ptr(table, "table", _bf16_types()),
        _ptr(ids, "ids", (torch.int32,), allow_none=True), C,
        _ptr(out_ids, "out_ids", (torch.int32,)),
        _ptr(out_logit, "out_logit", (torch.float32,), allow_none=True),
        _ptr(ws, "ws", (torch.int64, torch.uint8, torch.int32)), ws.numel() * ws.element_size(),
        _stream(stream), ctypes.byref(cfg)), "mtp_draft_argmax")


def mtp_verify_accept(hidden, head, draft, B: int, k: int, out_argmax, out_accept, out_tokens,
                      out_logit=None, ws=None, stream=None, path: int = MTP_PATH_AUTO,
                      blocks_per_cu: int = 0) -> None:
    """Verify GEMM + per-row argmax + greedy acceptance (see include/mtp.h)."""
    torch = _torch()
    Mv, H = hidden.shape
    V, H2 = head.shape
    if H != H2 or Mv != B * (k + 1):
        raise ValueError("hidden must be [B*(k+1)][H] with the head's H")
    if out_argmax.numel() != Mv or out_tokens.numel() != Mv or out_accept.numel() != B:
        raise ValueError("output sizes do not match B and k")
    if draft is not None and draft.numel() != B * k:
        raise ValueError("draft must be [B][k]")
    if ws is None:
        _no_alloc_in_capture("mtp_verify_accept")
        ws = alloc_workspace(mtp_verify_workspace_bytes(B, k, V, H), hidden.device, stream)
    cfg = _cfg(path, blocks_per_cu)
    _check(lib.mtp_verify_accept_cfg(
        _ptr(hidden, "hidden", _bf16_types()), B, k, H, _ptr(head, "head", _bf16_types()), V,
        _ptr(draft, "draft", (torch.int32,), allow_none=(k == 0)),
        _ptr(out_argmax, "out_argmax", (torch.int32,)),
        _ptr(out_logit, "out_logit", (torch.float32,), allow_none=True),
        _ptr(out_accept, "out_accept", (torch.int32,)),
        _ptr(out_tokens, "out_tokens", (torch.int32,)),
        _ptr(ws, "ws", (torch.int64, torch.uint8, torch.int32)), ws.numel() * ws.element_size(),
        _stream(stream), ctypes.byref(cfg)), "mtp_verify_accept")


def mtp_verify_accept_noalloc(hidden, head, draft, B: int, k: int, out_argmax, out_accept,
                              out_tokens, out_logit=None, stream=None) -> None:
    """mtp_verify_accept without a workspace: the library's static per-device
    scratch holds the counters (B*(k+1) <= MTP_NOALLOC_MAX_ROWS; calls that
    overlap on one GPU race, see include/mtp.h). Allocates nothing."""
    torch = _torch()
    Mv, H = hidden.shape
    V, H2 = head.shape
    if H != H2 or Mv != B * (k + 1):
        raise ValueError("hidden must be [B*(k+1)][H] with the head's H")
    if out_argmax.numel() != Mv or out_tokens.numel() != Mv or out_accept.numel() != B:
        raise ValueError("output sizes do not match B and k")
    if draft is not None and draft.numel() != B * k:
        raise ValueError("draft must be [B][k]")
    _check(lib.mtp_verify_accept_noalloc(
        _ptr(hidden, "hidden", _bf16_types()), B, k, H, _ptr(head, "head", _bf16_types()), V,
        _ptr(draft, "draft", (torch.int32,), allow_none=(k == 0)),
        _ptr(out_argmax, "out_argmax", (torch.int32,)),
        _ptr(out_logit, "out_logit", (torch.float32,), allow_none=True),
        _ptr(out_accept, "out_accept", (torch.int32,)),
        _ptr(out_tokens, "out_tokens", (torch.int32,)), _stream(stream)),
        "mtp_verify_accept_noalloc")


# --- tiled tables -------------------------------------------------------------

def mtp_tiled_bytes(rows: int, H: int) -> int:
    return int(lib.mtp_tiled_bytes(rows, H))


def alloc_tiled(rows: int, H: int, device=None):
    """Device buffer (uint8) sized for a tiled table of `rows` rows."""
    torch = _torch()
    n = mtp_tiled_bytes(rows, H)
    if n == 0:
        raise ValueError("rows or H out of range")
    return torch.empty(n, dtype=torch.uint8, device=device or "cuda")


def mtp_pack_tiled(head, ids, tiled, C: Optional[int] = None, stream=None) -> None:
    """Lay out rows ids[i] of the row-major head (or, ids None, its first C
    rows) in the tiled layout of include/mtp.h."""
    torch = _torch()
    V, H = head.shape
    if ids is not None:
        C = ids.numel()
    elif C is None:
        C = V
    _check(lib.mtp_pack_tiled(_ptr(head, "head", _bf16_types()), V, H,
                              _ptr(ids, "ids", (torch.int32,), allow_none=True), C,
                              _ptr(tiled, "tiled", (torch.uint8, torch.int16, torch.int32)),
                              tiled.numel() * tiled.element_size(), _stream(stream)),
           "mtp_pack_tiled")


def mtp_draft_argmax_tiled(hidden, table_tiled, C: int, ids, out_ids, out_logit=None, ws=None,
                           stream=None, blocks_per_cu: int = 0) -> None:
    """Draft GEMV + argmax over a tiled candidate table of C rows."""
    torch = _torch()
    M, H = hidden.shape
    if table_tiled.numel() * table_tiled.element_size() < mtp_tiled_bytes(C, H):
        raise ValueError("tiled table smaller than mtp_tiled_bytes(C, H)")
    if ids is not None and ids.numel() != C:
        raise ValueError("ids must have C entries")
    if out_ids.numel() != M or (out_logit is not None and out_logit.numel() != M):
        raise ValueError("outputs must have M entries")
    if ws is None:
        ws = alloc_workspace(mtp_draft_workspace_bytes(M, C, H), hidden.device, stream)
    cfg = _cfg(MTP_PATH_AUTO, blocks_per_cu)
    _check(lib.mtp_draft_argmax_tiled_cfg(
        _ptr(hidden, "hidden", _bf16_types()), M, H,
        _ptr(table_tiled, "table_tiled", (torch.uint8, torch.int16, torch.int32)),
        _ptr(ids, "ids", (torch.int32,), allow_none=True), C,
        _ptr(out_ids, "out_ids", (torch.int32,)),
        _ptr(out_logit, "out_logit", (torch.float32,), allow_none=True),
        _ptr(ws, "ws", (torch.int64, torch.uint8, torch.int32)), ws.numel() * ws.element_size(),
        _stream(stream), ctypes.byref(cfg)), "mtp_draft_argmax_tiled")


def mtp_verify_accept_tiled(hidden, head_tiled, V: int, draft, B: int, k: int, out_argmax,
                            out_accept, out_tokens, out_logit=None, ws=None, stream=None,
                            blocks_per_cu: int = 0) -> None:
    """Verify GEMM + argmax + acceptance over a tiled head of V rows."""
    torch = _torch()
    Mv, H = hidden.shape
    if Mv != B * (k + 1):
        raise ValueError("hidden must be [B*(k+1)][H]")
    if head_tiled.numel() * head_tiled.element_size() < mtp_tiled_bytes(V, H):
        raise ValueError("tiled head smaller than mtp_tiled_bytes(V, H)")
    if out_argmax.numel() != Mv or out_tokens.numel() != Mv or out_accept.numel() != B:
        raise ValueError("output sizes do not match B and k")
    if draft is not None and draft.numel() != B * k:
        raise ValueError("draft must be [B][k]")
    if ws is None:
        ws = alloc_workspace(mtp_verify_workspace_bytes(B, k, V, H), hidden.device, stream)
    cfg = _cfg(MTP_PATH_AUTO, blocks_per_cu)
    _check(lib.mtp_verify_accept_tiled_cfg(
        _ptr(hidden, "hidden", _bf16_types()), B, k, H,
        _ptr(head_tiled, "head_tiled", (torch.uint8, torch.int16, torch.int32)), V,
        _ptr(draft, "draft", (torch.int32,), allow_none=(k == 0)),
        _ptr(out_argmax, "out_argmax", (torch.int32,)),
        _ptr(out_logit, "out_logit", (torch.float32,), allow_none=True),
        _ptr(out_accept, "out_accept", (torch.int32,)),
        _ptr(out_tokens, "out_tokens", (torch.int32,)),
        _ptr(ws, "ws", (torch.int64, torch.uint8, torch.int32)), ws.numel() * ws.element_size(),
        _stream(stream), ctypes.byref(cfg)), "mtp_verify_accept_tiled")


def mtp_draft_argmax_gather(hidden, head, ids, out_ids, out_logit=None, ws=None, stream=None,
                            path: int = MTP_PATH_AUTO, blocks_per_cu: int = 0) -> None:
    """Draft over gathered candidates: out_ids[m] = the id in ``ids`` (any
    order; ids outside [0, V) skipped) maximising hidden[m] . head[id]."""
    torch = _torch()
    M, H = hidden.shape
    V, H2 = head.shape
    if H != H2:
        raise ValueError("hidden and head widths differ")
    C = ids.numel()
    if out_ids.numel() != M or (out_logit is not None and out_logit.numel() != M):
        raise ValueError("outputs must have M entries")
    if ws is None:
        _no_alloc_in_capture("mtp_draft_argmax_gather")
        ws = alloc_workspace(mtp_draft_workspace_bytes(M, C, H), hidden.device, stream)
    cfg = _cfg(path, blocks_per_cu)
    _check(lib.mtp_draft_argmax_gather_cfg(
        _ptr(hidden, "hidden", _bf16_types()), M, H, _ptr(head, "head", _bf16_types()), V,
        _ptr(ids, "ids", (torch.int32,)), C,
        _ptr(out_ids, "out_ids", (torch.int32,)),
        _ptr(out_logit, "out_logit", (torch.float32,), allow_none=True),
        _ptr(ws, "ws", (torch.int64, torch.uint8, torch.int32)), ws.numel() * ws.element_size(),
        _stream(stream), ctypes.byref(cfg)), "mtp_draft_argmax_gather")


# ---- FP8 candidate table -----------------------------------------------------


def mtp_fp8_table_bytes(C: int, H: int) -> int:
    return int(lib.mtp_fp8_table_bytes(C, H))


def mtp_pack_candidates_fp8(head, ids, table_q, scales, C: Optional[int] = None,
                            stream=None) -> None:
    """Quantise head rows ids (None: the first C rows) into E4M3 codes
    table_q [C][H] (uint8) and power-of-two row scales (float32 [C])."""
    torch = _torch()
    V, H = head.shape
    C = ids.numel() if ids is not None else (V if C is None else C)
    if tuple(table_q.shape) != (C, H) or scales.numel() != C:
        raise ValueError("table_q must be [C][H] and scales [C]")
    _check(lib.mtp_pack_candidates_fp8(
        _ptr(head, "head", _bf16_types()), V, H, _ptr(ids, "ids", (torch.int32,), allow_none=True),
        C, _ptr(table_q, "table_q", (torch.uint8,)), _ptr(scales, "scales", (torch.float32,)),
        _stream(stream)), "mtp_pack_candidates_fp8")


def mtp_draft_argmax_fp8(hidden, table_q, scales, ids, out_ids, out_logit=None, ws=None,
                         stream=None, path: int = MTP_PATH_AUTO, blocks_per_cu: int = 0) -> None:
    """Draft over an fp8 candidate table (see include/mtp.h)."""
    torch = _torch()
    M, H = hidden.shape
    C, H2 = table_q.shape
    if H != H2 or scales.numel() != C:
        raise ValueError("shapes differ")
    if ids is not None and ids.numel() != C:
        raise ValueError("ids must have C entries")
    if out_ids.numel() != M or (out_logit is not None and out_logit.numel() != M):
        raise ValueError("outputs must have M entries")
    if ws is None:
        _no_alloc_in_capture("mtp_draft_argmax_fp8")
        ws = alloc_workspace(mtp_draft_workspace_bytes(M, C, H), hidden.device, stream)
    cfg = _cfg(path, blocks_per_cu)
    _check(lib.mtp_draft_argmax_fp8_cfg(
        _ptr(hidden, "hidden", _bf16_types()), M, H, _ptr(table_q, "table_q", (torch.uint8,)),
        _ptr(scales, "scales", (torch.float32,)),
        _ptr(ids, "ids", (torch.int32,), allow_none=True), C,
        _ptr(out_ids, "out_ids", (torch.int32,)),
        _ptr(out_logit, "out_logit", (torch.float32,), allow_none=True),
        _ptr(ws, "ws", (torch.int64, torch.uint8, torch.int32)), ws.numel() * ws.element_size(),
        _stream(stream), ctypes.byref(cfg)), "mtp_draft_argmax_fp8")


def mtp_mxfp4_table_bytes(C: int, H: int) -> int:
    return int(lib.mtp_mxfp4_table_bytes(C, H))


def mtp_mxfp4_scale_bytes(C: int, H: int) -> int:
    return int(lib.mtp_mxfp4_scale_bytes(C, H))


MTP_MX_SCALE_OCP = 0
MTP_MX_SCALE_FIT = 1
MX_SCALE_RULES = {"ocp": MTP_MX_SCALE_OCP, "fit": MTP_MX_SCALE_FIT}


def mtp_pack_candidates_mxfp4(head, ids, table_q, scales, C: Optional[int] = None,
                              stream=None, rule: int = MTP_MX_SCALE_OCP) -> None:
    """Quantise head rows ids (None: the first C rows) to MXFP4: packed E2M1
    codes table_q [C][H/2] and E8M0 block scales [C][H/32] (both uint8), block
    scales by the OCP rule or the fit rule (MTP_MX_SCALE_*)."""
    torch = _torch()
    V, H = head.shape
    C = ids.numel() if ids is not None else (V if C is None else C)
    if tuple(table_q.shape) != (C, H // 2) or tuple(scales.shape) != (C, H // 32):
        raise ValueError("table_q must be [C][H/2] and scales [C][H/32]")
    _check(lib.mtp_pack_candidates_mxfp4_rule(
        _ptr(head, "head", _bf16_types()), V, H, _ptr(ids, "ids", (torch.int32,), allow_none=True),
        C, _ptr(table_q, "table_q", (torch.uint8,)), _ptr(scales, "scales", (torch.uint8,)),
        int(rule), _stream(stream)), "mtp_pack_candidates_mxfp4_rule")


def mtp_draft_argmax_mxfp4(hidden, table_q, scales, ids, out_ids, out_logit=None, ws=None,
                           stream=None, path: int = MTP_PATH_AUTO, blocks_per_cu: int = 0) -> None:
    """Draft over an MXFP4 candidate table (see include/mtp.h)."""
    torch = _torch()
    M, H = hidden.shape
    C, H2 = table_q.shape
    if 2 * H2 != H or tuple(scales.shape) != (C, H // 32):
        raise ValueError("shapes differ")
    if ids is not None and ids.numel() != C:
        raise ValueError("ids must have C entries")
    if out_ids.numel() != M or (out_logit is not None and out_logit.numel() != M):
        raise ValueError("outputs must have M entries")
    if ws is None:
        _no_alloc_in_capture("mtp_draft_argmax_mxfp4")
        ws = alloc_workspace(mtp_draft_workspace_bytes(M, C, H), hidden.device, stream)
    cfg = _cfg(path, blocks_per_cu)
    _check(lib.mtp_draft_argmax_mxfp4_cfg(
        _ptr(hidden, "hidden", _bf16_types()), M, H, _ptr(table_q, "table_q", (torch.uint8,)),
        _ptr(scales, "scales", (torch.uint8,)),
        _ptr(ids, "ids", (torch.int32,), allow_none=True), C,
        _ptr(out_ids, "out_ids", (torch.int32,)),
        _ptr(out_logit, "out_logit", (torch.float32,), allow_none=True),
        _ptr(ws, "ws", (torch.int64, torch.uint8, torch.int32)), ws.numel() * ws.element_size(),
        _stream(stream), ctypes.byref(cfg)), "mtp_draft_argmax_mxfp4")


def mtp_draft_argmax_fp8_gather(hidden, head_q, head_scales, ids, out_ids, out_logit=None,
                                ws=None, stream=None, path: int = MTP_PATH_AUTO,
                                blocks_per_cu: int = 0) -> None:
    """Draft over a candidate id list on an fp8 head (see include/mtp.h)."""
    torch = _torch()
    M, H = hidden.shape
    V, H2 = head_q.shape
    if H2 != H or tuple(head_scales.shape) != (V,):
        raise ValueError("shapes differ")
    C = ids.numel()
    if out_ids.numel() != M or (out_logit is not None and out_logit.numel() != M):
        raise ValueError("outputs must have M entries")
    if ws is None:
        _no_alloc_in_capture("mtp_draft_argmax_fp8_gather")
        ws = alloc_workspace(mtp_draft_workspace_bytes(M, C, H), hidden.device, stream)
    cfg = _cfg(path, blocks_per_cu)
    _check(lib.mtp_draft_argmax_fp8_gather_cfg(
        _ptr(hidden, "hidden", _bf16_types()), M, H, _ptr(head_q, "head_q", (torch.uint8,)),
        _ptr(head_scales, "head_scales", (torch.float32,)), V,
        _ptr(ids, "ids", (torch.int32,)), C,
        _ptr(out_ids, "out_ids", (torch.int32,)),
        _ptr(out_logit, "out_logit", (torch.float32,), allow_none=True),
        _ptr(ws, "ws", (torch.int64, torch.uint8, torch.int32)), ws.numel() * ws.element_size(),
        _stream(stream), ctypes.byref(cfg)), "mtp_draft_argmax_fp8_gather")


def mtp_draft_argmax_mxfp4_gather(hidden, head_q, head_scales, ids, out_ids, out_logit=None,
                                  ws=None, stream=None, path: int = MTP_PATH_AUTO,
                                  blocks_per_cu: int = 0) -> None:
    """Draft over a candidate id list on an MXFP4 head (see include/mtp.h)."""
    torch = _torch()
    M, H = hidden.shape
    V, H2 = head_q.shape
    if 2 * H2 != H or tuple(head_scales.shape) != (V, H // 32):
        raise ValueError("shapes differ")
    C = ids.numel()
    if out_ids.numel() != M or (out_logit is not None and out_logit.numel() != M):
        raise ValueError("outputs must have M entries")
    if ws is None:
        _no_alloc_in_capture("mtp_draft_argmax_mxfp4_gather")
        ws = alloc_workspace(mtp_draft_workspace_bytes(M, C, H), hidden.device, stream)
    cfg = _cfg(path, blocks_per_cu)
    _check(lib.mtp_draft_argmax_mxfp4_gather_cfg(
        _ptr(hidden, "hidden", _bf16_types()), M, H, _ptr(head_q, "head_q", (torch.uint8,)),
        _ptr(head_scales, "head_scales", (torch.uint8,)), V,
        _ptr(ids, "ids", (torch.int32,)), C,
        _ptr(out_ids, "out_ids", (torch.int32,)),
        _ptr(out_logit, "out_logit", (torch.float32,), allow_none=True),
        _ptr(ws, "ws", (torch.int64, torch.uint8, torch.int32)), ws.numel() * ws.element_size(),
        _stream(stream), ctypes.byref(cfg)), "mtp_draft_argmax_mxfp4_gather")


def mtp_tiled_mxfp4_bytes(rows: int, H: int) -> int:
    return int(lib.mtp_tiled_mxfp4_bytes(rows, H))


def mtp_tiled_mxfp4_scale_bytes(rows: int, H: int) -> int:
    return int(lib.mtp_tiled_mxfp4_scale_bytes(rows, H))


def alloc_tiled_mxfp4(rows: int, H: int, device=None):
    """uint8 buffers for an MXFP4 tiled table of `rows` rows: codes, scales."""
    torch = _torch()
    n = mtp_tiled_mxfp4_bytes(rows, H)
    if n == 0:
        raise ValueError("unsupported MXFP4 tiled shape")
    return (torch.empty(n, dtype=torch.uint8, device=device or "cuda"),
            torch.empty(mtp_tiled_mxfp4_scale_bytes(rows, H), dtype=torch.uint8,
                        device=device or "cuda"))


def mtp_pack_tiled_mxfp4(head, ids, tiled_q, tiled_scales, C: Optional[int] = None,
                         stream=None, rule: int = MTP_MX_SCALE_OCP) -> None:
    torch = _torch()
    V, H = head.shape
    C = ids.numel() if ids is not None else (V if C is None else C)
    _check(lib.mtp_pack_tiled_mxfp4_rule(
        _ptr(head, "head", _bf16_types()), V, H, _ptr(ids, "ids", (torch.int32,), allow_none=True),
        C, _ptr(tiled_q, "tiled_q", (torch.uint8,)), tiled_q.numel(),
        _ptr(tiled_scales, "tiled_scales", (torch.uint8,)), tiled_scales.numel(),
        int(rule), _stream(stream)), "mtp_pack_tiled_mxfp4_rule")


def mtp_draft_argmax_tiled_mxfp4(hidden, table_q, tiled_scales, C: int, ids, out_ids,
                                 out_logit=None, ws=None, stream=None,
                                 path: int = MTP_PATH_AUTO, blocks_per_cu: int = 0) -> None:
    """Draft over an MXFP4 tiled candidate table of C rows (matrix cores)."""
    torch = _torch()
    M, H = hidden.shape
    if table_q.numel() < mtp_tiled_mxfp4_bytes(C, H) or \
            tiled_scales.numel() < mtp_tiled_mxfp4_scale_bytes(C, H):
        raise ValueError("tiled table smaller than C rows")
    if ids is not None and ids.numel() != C:
        raise ValueError("ids must have C entries")
    if out_ids.numel() != M or (out_logit is not None and out_logit.numel() != M):
        raise ValueError("outputs must have M entries")
    if ws is None:
        _no_alloc_in_capture("mtp_draft_argmax_tiled_mxfp4")
        ws = alloc_workspace(mtp_draft_workspace_bytes(M, C, H), hidden.device, stream)
    cfg = _cfg(path, blocks_per_cu)
    _check(lib.mtp_draft_argmax_tiled_mxfp4_cfg(
        _ptr(hidden, "hidden", _bf16_types()), M, H, _ptr(table_q, "table_q", (torch.uint8,)),
        _ptr(tiled_scales, "tiled_scales", (torch.uint8,)),
        _ptr(ids, "ids", (torch.int32,), allow_none=True), C,
        _ptr(out_ids, "out_ids", (torch.int32,)),
        _ptr(out_logit, "out_logit", (torch.float32,), allow_none=True),
        _ptr(ws, "ws", (torch.int64, torch.uint8, torch.int32)), ws.numel() * ws.element_size(),
        _stream(stream), ctypes.byref(cfg)), "mtp_draft_argmax_tiled_mxfp4")


def mtp_tiled_fp8_bytes(rows: int, H: int) -> int:
    return int(lib.mtp_tiled_fp8_bytes(rows, H))


def alloc_tiled_fp8(rows: int, H: int, device=None):
    """A uint8 buffer for an fp8 tiled table of `rows` rows, and its scales."""
    torch = _torch()
    n = mtp_tiled_fp8_bytes(rows, H)
    if n == 0:
        raise ValueError("unsupported fp8 tiled shape")
    return (torch.empty(n, dtype=torch.uint8, device=device or "cuda"),
            torch.empty(rows, dtype=torch.float32, device=device or "cuda"))


def mtp_pack_tiled_fp8(head, ids, tiled_q, scales, C: Optional[int] = None, stream=None) -> None:
    torch = _torch()
    V, H = head.shape
    C = ids.numel() if ids is not None else (V if C is None else C)
    if scales.numel() != C:
        raise ValueError("scales must have C entries")
    _check(lib.mtp_pack_tiled_fp8(
        _ptr(head, "head", _bf16_types()), V, H, _ptr(ids, "ids", (torch.int32,), allow_none=True),
        C, _ptr(tiled_q, "tiled_q", (torch.uint8,)), tiled_q.numel(),
        _ptr(scales, "scales", (torch.float32,)), _stream(stream)), "mtp_pack_tiled_fp8")


def mtp_draft_argmax_tiled_fp8(hidden, table_q, scales, C: int, ids, out_ids, out_logit=None,
                               ws=None, stream=None, path: int = MTP_PATH_AUTO,
                               blocks_per_cu: int = 0) -> None:
    """Draft over an fp8 tiled candidate table of C rows (matrix cores)."""
    torch = _torch()
    M, H = hidden.shape
    if scales.numel() != C or (ids is not None and ids.numel() != C):
        raise ValueError("scales and ids must have C entries")
    if out_ids.numel() != M or (out_logit is not None and out_logit.numel() != M):
        raise ValueError("outputs must have M entries")
    if ws is None:
        _no_alloc_in_capture("mtp_draft_argmax_tiled_fp8")
        ws = alloc_workspace(mtp_draft_workspace_bytes(M, C, H), hidden.device, stream)
    cfg = _cfg(path, blocks_per_cu)
    _check(lib.mtp_draft_argmax_tiled_fp8_cfg(
        _ptr(hidden, "hidden", _bf16_types()), M, H, _ptr(table_q, "table_q", (torch.uint8,)),
        _ptr(scales, "scales", (torch.float32,)),
        _ptr(ids, "ids", (torch.int32,), allow_none=True), C,
        _ptr(out_ids, "out_ids", (torch.int32,)),
        _ptr(out_logit, "out_logit", (torch.float32,), allow_none=True),
        _ptr(ws, "ws", (torch.int64, torch.uint8, torch.int32)), ws.numel() * ws.element_size(),
        _stream(stream), ctypes.byref(cfg)), "mtp_draft_argmax_tiled_fp8")


# ---- streaming-read reference ----------------------------------------------

MTP_STREAM_SINK_WORDS = 8192


def mtp_stream_read(buf, sink, nbytes: Optional[int] = None, stream=None) -> None:
    """One plain streaming read of buf's first nbytes bytes (all of it by
    default); sink: int32/uint8 device tensor of MTP_STREAM_SINK_WORDS words."""
    torch = _torch()
    n = buf.numel() * buf.element_size() if nbytes is None else int(nbytes)
    if n > buf.numel() * buf.element_size():
        raise ValueError("nbytes exceeds the buffer")
    if sink.numel() * sink.element_size() < 4 * MTP_STREAM_SINK_WORDS:
        raise ValueError("sink too small")
    _check(lib.mtp_stream_read(_ptr(buf, "buf", (buf.dtype,)), n,
                               _ptr(sink, "sink", (torch.int32, torch.uint8)), _stream(stream)),
           "mtp_stream_read")


MTP_PROBE_MAX_WGS = 4096
MTP_PROBE_MAX_ITERS = 1024


def mtp_probe_atomic(words, ticks, wgs: int, iters: int, same: bool = False, stream=None) -> None:
    """Atomic round-trip probe: in each of wgs workgroups one lane runs iters
    dependent agent-scope fetch-and-adds on its own word of words (int32 device
    tensor of 64 * wgs words) or all on words[0] (same); ticks (int64 device
    tensor of wgs) gets each chain's 100 MHz tick count in its low 63 bits."""
    torch = _torch()
    need = 2 if same else 64 * wgs
    if words.numel() * words.element_size() < 4 * need:
        raise ValueError("words too small")
    if ticks.numel() * ticks.element_size() < 8 * wgs:
        raise ValueError("ticks too small")
    _check(lib.mtp_probe_atomic(_ptr(words, "words", (torch.int32,)), int(wgs), int(iters),
                                1 if same else 0, _ptr(ticks, "ticks", (torch.int64,)),
                                _stream(stream)),
           "mtp_probe_atomic")


# ---- graph-captured MTP step ----------------------------------------------


class Graph:
    """One captured MTP step (``mtp_graph_begin`` / ``mtp_graph_end``).

    Capture on a created (non-null) stream::

        g = Graph()
        with torch.cuda.stream(s):
            g.begin()
            mtp_draft_argmax(...); ...; mtp_verify_accept(...)
            g.end()
            g.launch()          # replays the step on the current stream

    Every buffer passed during capture must stay allocated until ``destroy``;
    allocate all of them before ``begin``.
    """

    def __init__(self):
        self._h = _null_handle()

    def begin(self, stream=None) -> None:
        global _capturing
        _check(lib.mtp_graph_begin(_stream(stream)), "mtp_graph_begin")
        _capturing += 1

    def end(self, stream=None) -> None:
        global _capturing
        _capturing = max(0, _capturing - 1)
        h = _null_handle()
        _check(lib.mtp_graph_end(_stream(stream), ctypes.byref(h)), "mtp_graph_end")
        self.destroy()
        self._h = h

    def launch(self, stream=None) -> None:
        if not self._h:
            raise MTPError(MTP_ERR_INVALID_ARG, "mtp_graph_launch (no captured graph)")
        _check(lib.mtp_graph_launch(self._h, _stream(stream)), "mtp_graph_launch")

    def destroy(self) -> None:
        if self._h:
            lib.mtp_graph_destroy(self._h)
            self._h = _null_handle()

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def _null_handle():
    return ctypes.c_void_p()
