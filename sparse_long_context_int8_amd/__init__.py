"""Python binding of libspmla.so, the MI355X sparse-MLA prefill library.

Argument marshalling only: every step of the layer runs in the library's HIP
kernels. torch supplies device memory and the current stream. Function names
match the C ABI in include/spmla.h.

If the shared library is missing it is built once with hipcc; if it cannot be
built or loaded, importing the entry points raises instead of falling back to
any other implementation.
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = [
    "SpmlaError",
    "spmla_desc",
    "make_desc",
    "load_library",
    "spmla_abi_version",
    "spmla_check_desc",
    "spmla_num_bands",
    "spmla_indexer_scores",
    "spmla_topk",
    "spmla_sparse_attn",
    "spmla_sparse_attn_grouped",
    "spmla_compress",
    "spmla_prefill_workspace_bytes",
    "spmla_prefill",
    "spmla_prefill_noalloc",
    "prefill",
    "EXPORTED_SYMBOLS",
]

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libspmla.so")

SPMLA_OK = 0
SPMLA_EINVAL = -1
SPMLA_EUNSUPPORTED = -2
SPMLA_EWORKSPACE = -3
SPMLA_EHIP = -4

EXPORTED_SYMBOLS = [
    "spmla_last_error",
    "spmla_abi_version",
    "spmla_check_desc",
    "spmla_num_bands",
    "spmla_indexer_scores",
    "spmla_topk",
    "spmla_sparse_attn",
    "spmla_sparse_attn_grouped",
    "spmla_compress",
    "spmla_prefill_workspace_bytes",
    "spmla_prefill",
    "spmla_prefill_noalloc",
]


class SpmlaError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"spmla error {code}: {message}")
        self.code = code


class spmla_desc(ctypes.Structure):
    _fields_ = [
        ("n_q", ctypes.c_int32),
        ("q_pos0", ctypes.c_int32),
        ("n_raw", ctypes.c_int32),
        ("n_comp", ctypes.c_int32),
        ("ratio", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("band", ctypes.c_int32),
        ("n_heads", ctypes.c_int32),
        ("d_qk", ctypes.c_int32),
        ("d_v", ctypes.c_int32),
        ("idx_heads", ctypes.c_int32),
        ("idx_dim", ctypes.c_int32),
        ("scale", ctypes.c_float),
    ]


def make_desc(n_q, q_pos0, window, top_k, *, ratio=4, band=2048, n_heads=16, d_qk=576, d_v=512,
              idx_heads=4, idx_dim=64, scale=None, n_raw=None, n_comp=None) -> spmla_desc:
    n_raw = q_pos0 + n_q if n_raw is None else n_raw
    n_comp = n_raw // ratio if n_comp is None else n_comp
    scale = 1.0 / math.sqrt(d_qk) if scale is None else scale
    return spmla_desc(n_q, q_pos0, n_raw, n_comp, ratio, window, top_k, band, n_heads, d_qk, d_v,
                      idx_heads, idx_dim, scale)


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libspmla.so (building it first if it does not exist)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        from . import build as _build

        _build.build()
    if not os.path.exists(path):
        raise ImportError(f"libspmla.so not found at {path}")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    D = ctypes.POINTER(spmla_desc)
    sig = {
        "spmla_last_error": (ctypes.c_char_p, []),
        "spmla_abi_version": (ctypes.c_int, []),
        "spmla_check_desc": (ctypes.c_int, [D]),
        "spmla_num_bands": (ctypes.c_int, [D]),
        "spmla_indexer_scores": (ctypes.c_int, [D, P, P, P, P, P]),
        "spmla_topk": (ctypes.c_int, [D, P, P, P, P]),
        "spmla_sparse_attn": (ctypes.c_int, [D, P, P, P, P, P, P, P]),
        "spmla_sparse_attn_grouped": (ctypes.c_int, [D, P, P, P, P, P, P, P]),
        "spmla_compress": (ctypes.c_int, [D, P, P, ctypes.c_int32, P]),
        "spmla_prefill_workspace_bytes": (ctypes.c_int, [D, ctypes.POINTER(ctypes.c_size_t)]),
        "spmla_prefill": (ctypes.c_int, [D, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]),
        "spmla_prefill_noalloc": (ctypes.c_int, [D, P, P, P, P, P, P, P, P, P, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(rc: int) -> int:
    if rc < 0:
        msg = load_library().spmla_last_error().decode(errors="replace")
        raise SpmlaError(rc, msg)
    return rc


def _validate(t, dtype=None, name="tensor", numel=0):
    """dtype, layout and element count of one argument. The library sees
    only pointers, so the count is checked here against `numel`, the count
    the descriptor implies: a short tensor raises instead of reaching a
    kernel."""
    if t is None or isinstance(t, int):
        return
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, the descriptor needs {numel}")


def _addr(t, name):
    """Device pointer of an argument _validate has accepted (None -> NULL; an
    int is a raw address, used by tests of the C checks)."""
    if t is None:
        return None
    if isinstance(t, int):
        return ctypes.c_void_p(t)
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    return ctypes.c_void_p(t.data_ptr())


def _ptr(t, dtype=None, name="tensor", numel=0):
    """Device pointer of a contiguous device tensor, validated."""
    _validate(t, dtype, name, numel)
    return _addr(t, name)


def _ptrs(*specs):
    """Pointers of several arguments, each (tensor, dtype, name, numel):
    every argument is validated before any is looked up on the device."""
    for spec in specs:
        _validate(*spec)
    return [_addr(spec[0], spec[2]) for spec in specs]


# Element count of each argument as include/spmla.h lays it out, from the
# descriptor fields it needs (each field read of a ctypes structure costs
# host time on every call).
_COUNTS = {
    "q": lambda d: d.n_q * d.n_heads * d.d_qk,
    "kv_comp": lambda d: d.n_comp * d.d_qk,
    "kv_raw": lambda d: d.n_raw * d.d_qk,
    "iq": lambda d: d.n_q * d.idx_heads * d.idx_dim,
    "iw": lambda d: d.n_q * d.idx_heads,
    "ik": lambda d: d.n_comp * d.idx_dim,
    "scores": lambda d: d.n_q * d.n_comp,
    "sel": lambda d: d.n_q * d.top_k,
    "out": lambda d: d.n_q * d.n_heads * d.d_v,
    "lse": lambda d: d.n_q * d.n_heads,
}


def _n(desc, name: str) -> int:
    """Element count of an argument as include/spmla.h lays it out."""
    return _COUNTS[name](desc)


def _attn_ptrs(desc, q, kv_comp, kv_raw, sel, out, lse):
    torch = _dt()
    return _ptrs((q, torch.float16, "q", _n(desc, "q")), (kv_comp, torch.float16, "kv_comp", _n(desc, "kv_comp")),
                 (kv_raw, torch.float16, "kv_raw", _n(desc, "kv_raw")), (sel, torch.int32, "sel", _n(desc, "sel")),
                 (out, torch.float32, "out", _n(desc, "out")), (lse, torch.float32, "lse", _n(desc, "lse")))


def _stream(stream):
    if stream is None:
        import torch

        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _dt():
    import torch

    return torch


def spmla_abi_version() -> int:
    return load_library().spmla_abi_version()


def spmla_check_desc(desc: spmla_desc) -> int:
    return _check(load_library().spmla_check_desc(ctypes.byref(desc)))


def spmla_num_bands(desc: spmla_desc) -> int:
    return _check(load_library().spmla_num_bands(ctypes.byref(desc)))


def spmla_indexer_scores(desc, iq, iw, ik, scores, stream=None) -> None:
    torch = _dt()
    _check(load_library().spmla_indexer_scores(
        ctypes.byref(desc), *_ptrs((iq, torch.int8, "iq", _n(desc, "iq")), (iw, torch.int8, "iw", _n(desc, "iw")),
                                   (ik, torch.int8, "ik", _n(desc, "ik")),
                                   (scores, torch.int32, "scores", _n(desc, "scores"))),
        _stream(stream)))


def spmla_topk(desc, scores, sel, n_sel=None, stream=None) -> None:
    torch = _dt()
    _check(load_library().spmla_topk(
        ctypes.byref(desc), *_ptrs((scores, torch.int32, "scores", _n(desc, "scores")),
                                   (sel, torch.int32, "sel", _n(desc, "sel")), (n_sel, torch.int32, "n_sel", desc.n_q)),
        _stream(stream)))


def spmla_sparse_attn(desc, q, kv_comp, kv_raw, sel, out, lse=None, stream=None) -> None:
    torch = _dt()
    _check(load_library().spmla_sparse_attn(
        ctypes.byref(desc), *_attn_ptrs(desc, q, kv_comp, kv_raw, sel, out, lse), _stream(stream)))


def spmla_sparse_attn_grouped(desc, q, kv_comp, kv_raw, sel, out, lse=None, stream=None) -> None:
    torch = _dt()
    _check(load_library().spmla_sparse_attn_grouped(
        ctypes.byref(desc), *_attn_ptrs(desc, q, kv_comp, kv_raw, sel, out, lse), _stream(stream)))


def spmla_compress(desc, kv_raw, kv_comp, comp_begin=0, stream=None) -> None:
    torch = _dt()
    _check(load_library().spmla_compress(
        ctypes.byref(desc), *_ptrs((kv_raw, torch.float16, "kv_raw", _n(desc, "kv_raw")),
                                   (kv_comp, torch.float16, "kv_comp", _n(desc, "kv_comp"))),
        ctypes.c_int32(comp_begin), _stream(stream)))


def spmla_prefill_workspace_bytes(desc) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().spmla_prefill_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def spmla_prefill(desc, q, kv_comp, kv_raw, iq, iw, ik, out, lse, sel_out, workspace,
                  workspace_bytes=None, stream=None) -> None:
    torch = _dt()
    held = 0 if workspace is None or isinstance(workspace, int) else workspace.numel() * workspace.element_size()
    if workspace_bytes is None:
        workspace_bytes = held
    elif not isinstance(workspace, int) and workspace is not None and workspace_bytes > held:
        raise ValueError(f"workspace_bytes={workspace_bytes} exceeds the workspace tensor's {held} bytes")
    _check(load_library().spmla_prefill(
        ctypes.byref(desc),
        *_ptrs((q, torch.float16, "q", _n(desc, "q")), (kv_comp, torch.float16, "kv_comp", _n(desc, "kv_comp")),
               (kv_raw, torch.float16, "kv_raw", _n(desc, "kv_raw")), (iq, torch.int8, "iq", _n(desc, "iq")),
               (iw, torch.int8, "iw", _n(desc, "iw")), (ik, torch.int8, "ik", _n(desc, "ik")),
               (out, torch.float32, "out", _n(desc, "out")), (lse, torch.float32, "lse", _n(desc, "lse")),
               (sel_out, torch.int32, "sel_out", _n(desc, "sel")), (workspace, None, "workspace", 0)),
        ctypes.c_size_t(workspace_bytes), _stream(stream)))


def spmla_prefill_noalloc(desc, q, kv_comp, kv_raw, iq, iw, ik, out, lse, sel_out, stream=None) -> None:
    torch = _dt()
    _check(load_library().spmla_prefill_noalloc(
        ctypes.byref(desc),
        *_ptrs((q, torch.float16, "q", _n(desc, "q")), (kv_comp, torch.float16, "kv_comp", _n(desc, "kv_comp")),
               (kv_raw, torch.float16, "kv_raw", _n(desc, "kv_raw")), (iq, torch.int8, "iq", _n(desc, "iq")),
               (iw, torch.int8, "iw", _n(desc, "iw")), (ik, torch.int8, "ik", _n(desc, "ik")),
               (out, torch.float32, "out", _n(desc, "out")), (lse, torch.float32, "lse", _n(desc, "lse")),
               (sel_out, torch.int32, "sel_out", _n(desc, "sel"))),
        _stream(stream)))


def prefill(desc, dev: dict, want_sel=True, want_lse=True, stream=None):
    """Allocate outputs and workspace with torch and run spmla_prefill.

    `dev` holds device tensors q, kv_comp, kv_raw, iq, iw, ik. With a
    `stream` (a torch stream or a raw hipStream_t), outputs and workspace are
    allocated on that stream, so torch's allocator reuses the workspace only
    in that stream's order once this function drops it; the caller orders
    the inputs before the call and synchronizes before reading the outputs.
    Returns (out, lse or None, sel or None).
    """
    import contextlib

    torch = _dt()
    device = dev["q"].device
    if stream is None:
        ctx = contextlib.nullcontext()
    else:
        ts = torch.cuda.ExternalStream(stream) if isinstance(stream, int) else stream
        ctx = torch.cuda.stream(ts)
    with ctx:
        out = torch.empty((desc.n_q, desc.n_heads, desc.d_v), dtype=torch.float32, device=device)
        lse = torch.empty((desc.n_q, desc.n_heads), dtype=torch.float32, device=device) if want_lse else None
        sel = torch.empty((desc.n_q, desc.top_k), dtype=torch.int32, device=device) if want_sel else None
        nbytes = spmla_prefill_workspace_bytes(desc)
        ws = torch.empty((max(nbytes, 16),), dtype=torch.uint8, device=device)
        spmla_prefill(desc, dev["q"], dev["kv_comp"], dev["kv_raw"], dev["iq"], dev["iw"], dev["ik"],
                      out, lse, sel, ws, nbytes, stream)
    return out, lse, sel
