"""Thin ctypes binding of libpop (declared in include/pop.h).

Argument marshalling only: every step of the path runs in the HIP kernels of
libpop.so.  Importing this module loads the library and raises ImportError
when it has not been built (run ``python -m online_structured_ffn_amd.build``);
there is no fallback.  Tensors are torch tensors on the current HIP device;
work is enqueued on ``stream`` (default: torch's current stream).

libpop_debug.so, built beside libpop.so, validates the partition's index
lists on the host inside every entry point that takes them; select it for a
whole process with POP_LIBRARY, or for a block of calls with
``using_library(DEBUG_LIB_PATH)``.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import re

import numpy as np

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# POP_LIBRARY selects another build of the same library (e.g. a tuning variant).
LIB_PATH = os.environ.get("POP_LIBRARY") or os.path.join(_HERE, "libpop.so")
DEBUG_LIB_PATH = os.path.join(_HERE, "libpop_debug.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "pop.h")

POP_F32, POP_BF16 = 0, 1
_c_i32, _c_i64, _c_dbl, _c_size, _c_vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_double, ctypes.c_size_t, ctypes.c_void_p


class PopCounts(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("d_ff", "c_low", "c_high", "n_P", "n_C", "n_R", "n_live", "k")]


class LayerShape(ctypes.Structure):
    """pop_layer_shape."""
    _fields_ = [("d", ctypes.c_int32), ("n_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("d_ff", ctypes.c_int32), ("cache_len", ctypes.c_int32),
                ("eps", ctypes.c_double), ("rope_theta", ctypes.c_double)]


class LayerWeights(ctypes.Structure):
    """pop_layer_weights (device pointers)."""
    _fields_ = [(n, ctypes.c_void_p) for n in ("attn_norm", "Wqkv_T", "Wo_T", "ffn_norm", "W_gate", "W_up",
                                               "W_downT")]


class PopError(RuntimeError):
    def __init__(self, func, status, detail):
        self.status = status
        super().__init__(f"{func}: {status_string(status)}: {detail}")


_loaded: dict = {}


def _load(path: str = LIB_PATH):
    if path in _loaded:
        return _loaded[path]
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m online_structured_ffn_amd.build`")
    lib = ctypes.CDLL(path)
    sig = {
        "pop_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "pop_last_error": (ctypes.c_char_p, []),
        "pop_partition_counts": (ctypes.c_int, [_c_i32, _c_dbl, _c_dbl, ctypes.POINTER(PopCounts)]),
        "pop_decode_topk_count": (ctypes.c_int, [_c_i32, _c_dbl, _c_i32, _c_i32, ctypes.POINTER(_c_i32)]),
        "pop_check_lists": (ctypes.c_int, [_c_vp, _c_i32, _c_vp, _c_i32, _c_vp, _c_i32, _c_i32]),
        "pop_prefill_workspace_bytes": (_c_size, [_c_i64, _c_i32, _c_i32]),
        "pop_prefill_partition": (ctypes.c_int, [_c_vp, _c_i64, _c_i32, _c_vp, _c_i32, ctypes.c_int, _c_dbl, _c_dbl,
                                                 _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_size, _c_vp]),
        "pop_decode_workspace_bytes": (_c_size, [_c_i32, _c_i32, _c_i32]),
        "pop_decode_ffn": (ctypes.c_int, [_c_vp, _c_i32, _c_i32, _c_vp, _c_vp, _c_vp, _c_i32, ctypes.c_int,
                                          _c_vp, _c_i32, _c_vp, _c_i32, _c_dbl, _c_vp, _c_vp, _c_vp, _c_size, _c_vp]),
        "pop_dense_ffn_decode": (ctypes.c_int, [_c_vp, _c_i32, _c_i32, _c_vp, _c_vp, _c_vp, _c_i32, ctypes.c_int,
                                                _c_vp, _c_vp, _c_size, _c_vp]),
        "pop_decode_ffn_noalloc": (ctypes.c_int, [_c_vp, _c_i32, _c_i32, _c_vp, _c_vp, _c_vp, _c_i32, ctypes.c_int,
                                                  _c_vp, _c_i32, _c_vp, _c_i32, _c_dbl, _c_vp, _c_vp, _c_vp]),
        "pop_prefill_importance_workspace_bytes": (_c_size, [_c_i64, _c_i32, _c_i32]),
        "pop_prefill_importance": (ctypes.c_int, [_c_vp, _c_i64, _c_i32, _c_vp, _c_i32, ctypes.c_int, _c_vp, _c_vp,
                                                  _c_size, _c_vp]),
        "pop_partition_select": (ctypes.c_int, [_c_vp, _c_i32, _c_dbl, _c_dbl, _c_vp, _c_vp, _c_vp, _c_vp]),
        "pop_decode_gateup": (ctypes.c_int, [_c_vp, _c_i32, _c_i32, _c_vp, _c_vp, _c_i32, ctypes.c_int, _c_vp, _c_i32,
                                             _c_vp, _c_i32, _c_vp, _c_vp, _c_vp]),
        "pop_decode_select": (ctypes.c_int, [_c_vp, _c_i32, _c_vp, _c_i32, _c_vp, _c_vp, _c_vp]),
        "pop_decode_down_workspace_bytes": (_c_size, [_c_i32, _c_i32, _c_i32]),
        "pop_set_trace_events": (ctypes.c_int, [ctypes.POINTER(_c_vp), _c_i32]),
        "pop_trace_recorded": (_c_i32, []),
        "pop_hbm_read_probe": (ctypes.c_int, [_c_vp, _c_size, _c_vp, _c_i32, _c_vp]),
        "pop_dense_ffn_prefill_workspace_bytes": (_c_size, [_c_i64, _c_i32, _c_i32, ctypes.c_int]),
        "pop_moe_route_top2": (ctypes.c_int, [_c_vp, _c_i32, _c_i32, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp]),
        "pop_moe_prefill_workspace_bytes": (_c_size, [_c_i64, _c_i32, _c_i32, _c_i32]),
        "pop_moe_prefill_partition": (ctypes.c_int, [_c_vp, _c_i64, _c_i32, _c_vp, _c_i32, _c_vp, _c_i32, ctypes.c_int,
                                                     _c_dbl, _c_dbl, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_size,
                                                     _c_vp]),
        "pop_moe_decode_workspace_bytes": (_c_size, [_c_i32, _c_i32, _c_i32, _c_i32]),
        "pop_moe_decode_ffn": (ctypes.c_int, [_c_vp, _c_i32, _c_i32, _c_vp, _c_i32, _c_vp, _c_vp, _c_vp, _c_i32,
                                              ctypes.c_int, _c_vp, _c_i32, _c_vp, _c_i32, _c_dbl, _c_vp, _c_vp, _c_vp,
                                              _c_size, _c_vp]),
        "pop_dense_ffn_prefill": (ctypes.c_int, [_c_vp, _c_i64, _c_i32, _c_vp, _c_vp, _c_vp, _c_i32, ctypes.c_int,
                                                 _c_vp, _c_vp, _c_size, _c_vp]),
        "pop_prefill_ffn_partition_workspace_bytes": (_c_size, [_c_i64, _c_i32, _c_i32, ctypes.c_int]),
        "pop_prefill_ffn_partition": (ctypes.c_int, [_c_vp, _c_i64, _c_i32, _c_vp, _c_vp, _c_vp, _c_i32, ctypes.c_int,
                                                     _c_dbl, _c_dbl, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_size,
                                                     _c_vp]),
        "pop_decode_down": (ctypes.c_int, [_c_vp, _c_i32, _c_i32, _c_vp, _c_i32, _c_i32, ctypes.c_int, _c_vp, _c_i32,
                                           _c_vp, _c_vp, _c_i32, _c_vp, _c_vp, _c_size, _c_vp]),
        "pop_decode_periodic_workspace_bytes": (_c_size, [_c_i32, _c_i32, _c_i32]),
        "pop_decode_ffn_periodic": (ctypes.c_int, [_c_vp, _c_i32, _c_i32, _c_vp, _c_vp, _c_vp, _c_i32, ctypes.c_int,
                                                   _c_vp, _c_i32, _c_vp, _c_i32, _c_dbl, _c_i32, _c_i32, _c_vp, _c_vp,
                                                   _c_vp, _c_vp, _c_vp, _c_vp, _c_size, _c_vp]),
        "pop_layer_prefill_workspace_bytes": (_c_size, [_c_i32, _c_i32, ctypes.POINTER(LayerShape), ctypes.c_int]),
        "pop_layer_prefill": (ctypes.c_int, [_c_vp, _c_i32, _c_i32, ctypes.POINTER(LayerShape),
                                             ctypes.POINTER(LayerWeights), ctypes.c_int, _c_vp, _c_vp, _c_dbl, _c_dbl,
                                             _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_size, _c_vp]),
        "pop_layer_decode_workspace_bytes": (_c_size, [_c_i32, ctypes.POINTER(LayerShape), ctypes.c_int]),
        "pop_layer_decode": (ctypes.c_int, [_c_vp, _c_i32, ctypes.POINTER(LayerShape), ctypes.POINTER(LayerWeights),
                                            ctypes.c_int, _c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_vp, _c_i32, _c_dbl,
                                            _c_i32, _c_vp, _c_vp, _c_size, _c_vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _loaded[path] = lib
    return lib


lib = _load()


@contextlib.contextmanager
def using_library(path: str):
    """Route this module's calls through another build of libpop (loaded
    beside the default one) inside the block; not thread-safe."""
    global lib
    prev = lib
    lib = _load(path)
    try:
        yield lib
    finally:
        lib = prev


def _header_define(name: str) -> int:
    m = re.search(rf"^#define {name} (\d+)", open(HEADER).read(), re.M)
    if m is None:
        raise ImportError(f"{name} is not defined in {HEADER}")
    return int(m.group(1))


# Byte offset of z in a decode workspace (the bytes before it are control words).
DECODE_WS_Z_OFFSET = _header_define("POP_DECODE_WS_Z_OFFSET")


def declared_functions() -> list[str]:
    """Every function include/pop.h declares."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(pop_[a-z_0-9]+)\s*\(", text, re.M)))


def status_string(status: int) -> str:
    return lib.pop_status_string(int(status)).decode()


def _check(func: str, status: int):
    if status != 0:
        raise PopError(func, status, lib.pop_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dtype(t) -> int:
    if t.dtype == torch.float32:
        return POP_F32
    if t.dtype == torch.bfloat16:
        return POP_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous and on the GPU")


# ---------------------------------------------------------------- host-only
def pop_partition_counts(d_ff: int, r: float, gamma: float) -> dict:
    c = PopCounts()
    _check("pop_partition_counts", lib.pop_partition_counts(int(d_ff), float(r), float(gamma), ctypes.byref(c)))
    return {n: getattr(c, n) for n, _ in PopCounts._fields_}


def pop_check_lists(R, C, d_ff: int, P=None) -> None:
    """Host check of a partition's index lists (array-likes of channel ids):
    each strictly ascending in [0, d_ff), no channel in two lists.  Raises
    PopError naming the first violation."""
    arrs = [np.ascontiguousarray(np.asarray(a if a is not None else [], dtype=np.int64).ravel()) for a in (R, C, P)]
    if any(a.size and (a.min() < -2**31 or a.max() >= 2**31) for a in arrs):
        raise ValueError("channel ids must fit in int32")
    arrs = [a.astype(np.int32) for a in arrs]
    ptr = lambda a: ctypes.c_void_p(a.ctypes.data) if a.size else None
    _check("pop_check_lists", lib.pop_check_lists(ptr(arrs[0]), arrs[0].size, ptr(arrs[1]), arrs[1].size,
                                                  ptr(arrs[2]), arrs[2].size, int(d_ff)))


def pop_prefill_workspace_bytes(n_tokens: int, d: int, d_ff: int) -> int:
    return int(lib.pop_prefill_workspace_bytes(int(n_tokens), int(d), int(d_ff)))


def pop_decode_workspace_bytes(batch: int, d: int, d_ff: int) -> int:
    return int(lib.pop_decode_workspace_bytes(int(batch), int(d), int(d_ff)))


def workspace(nbytes: int, device=None) -> torch.Tensor:
    """A device workspace (zero-filled; the library does not require it)."""
    return torch.zeros(max(int(nbytes), 16), dtype=torch.uint8, device=device or "cuda")


# ---------------------------------------------------------------- device calls
def pop_prefill_partition(X, W_up, r: float, gamma: float, *, importance: bool = False, out=None,
                          ws=None, stream=None):
    """(R, C, P[, I]) for prompt activations X [n_tokens, d] and W_up [d_ff, d]."""
    _dev(X, W_up)
    n_tokens, d = X.shape
    d_ff = W_up.shape[0]
    if W_up.shape[1] != d or X.dtype != W_up.dtype:
        raise ValueError("X and W_up disagree in width or dtype")
    c = pop_partition_counts(d_ff, r, gamma)
    dev = W_up.device
    if out is None:
        R = torch.empty(c["n_R"], dtype=torch.int32, device=dev)
        C = torch.empty(c["n_C"], dtype=torch.int32, device=dev)
        P = torch.empty(c["n_P"], dtype=torch.int32, device=dev)
        I = torch.empty(d_ff, dtype=torch.float32, device=dev) if importance else None
    else:
        R, C, P, I = out
    if ws is None:
        ws = workspace(pop_prefill_workspace_bytes(n_tokens, d, d_ff), dev)
    _check("pop_prefill_partition", lib.pop_prefill_partition(
        _ptr(X), n_tokens, d, _ptr(W_up), d_ff, _dtype(W_up), float(r), float(gamma),
        _ptr(R), _ptr(C), _ptr(P), _ptr(I), _ptr(ws), ws.numel(), _stream(stream)))
    return (R, C, P, I) if importance else (R, C, P)


def pop_decode_ffn(x, W_gate, W_up, W_downT, R, C, r: float, *, y=None, selected: bool = False,
                   ws=None, stream=None):
    """y [batch, d] (fp32) for one decode step; optionally also the selected candidates."""
    _dev(x, W_gate, W_up, W_downT, R, C)
    batch, d = x.shape
    d_ff = W_gate.shape[0]
    dev = W_gate.device
    if y is None:
        y = torch.empty((batch, d), dtype=torch.float32, device=dev)
    S = None
    if selected:
        S = torch.empty(pop_decode_topk_count(d_ff, r, R.numel(), C.numel()), dtype=torch.int32, device=dev)
    if ws is None:
        ws = workspace(pop_decode_workspace_bytes(batch, d, d_ff), dev)
    _check("pop_decode_ffn", lib.pop_decode_ffn(
        _ptr(x), batch, d, _ptr(W_gate), _ptr(W_up), _ptr(W_downT), d_ff, _dtype(W_gate),
        _ptr(R), R.numel(), _ptr(C), C.numel(), float(r), _ptr(y), _ptr(S), _ptr(ws), ws.numel(),
        _stream(stream)))
    return (y, S) if selected else y


def pop_decode_ffn_noalloc(x, W_gate, W_up, W_downT, R, C, r: float, *, y=None, selected: bool = False,
                           stream=None):
    """pop_decode_ffn with the library's own device scratch as workspace (the
    C call allocates nothing; calls on one GPU must not overlap)."""
    _dev(x, W_gate, W_up, W_downT, R, C)
    batch, d = x.shape
    d_ff = W_gate.shape[0]
    dev = W_gate.device
    if y is None:
        y = torch.empty((batch, d), dtype=torch.float32, device=dev)
    S = None
    if selected:
        S = torch.empty(pop_decode_topk_count(d_ff, r, R.numel(), C.numel()), dtype=torch.int32, device=dev)
    _check("pop_decode_ffn_noalloc", lib.pop_decode_ffn_noalloc(
        _ptr(x), batch, d, _ptr(W_gate), _ptr(W_up), _ptr(W_downT), d_ff, _dtype(W_gate),
        _ptr(R), R.numel(), _ptr(C), C.numel(), float(r), _ptr(y), _ptr(S), _stream(stream)))
    return (y, S) if selected else y


class PeriodicState:
    """The state pop_decode_ffn_periodic carries between steps: the activation
    memory [n_C] (fp32, zero at the start), the current selection as
    positions into C and as channels [k], and the kept steps' rows [n_R + k]."""

    def __init__(self, d_ff: int, r: float, n_R: int, n_C: int, device):
        k = pop_decode_topk_count(d_ff, r, n_R, n_C)
        self.memory = torch.zeros(n_C, dtype=torch.float32, device=device)
        self.positions = torch.zeros(k, dtype=torch.int32, device=device)
        self.selected = torch.zeros(k, dtype=torch.int32, device=device)
        self.rows = torch.zeros(n_R + k, dtype=torch.int32, device=device)


def pop_decode_periodic_workspace_bytes(batch: int, d: int, d_ff: int) -> int:
    return int(lib.pop_decode_periodic_workspace_bytes(batch, d, d_ff))


def pop_decode_ffn_periodic(x, W_gate, W_up, W_downT, R, C, r: float, step: int, period: int,
                            state: "PeriodicState", *, y=None, ws=None, stream=None):
    """y [batch, d] (fp32) for decode step ``step`` of the periodic-refresh
    mode; ``state`` (memory, positions, selected) is read and updated."""
    _dev(x, W_gate, W_up, W_downT, R, C)
    batch, d = x.shape
    d_ff = W_gate.shape[0]
    dev = W_gate.device
    if y is None:
        y = torch.empty((batch, d), dtype=torch.float32, device=dev)
    if ws is None:
        ws = workspace(pop_decode_periodic_workspace_bytes(batch, d, d_ff), dev)
    _check("pop_decode_ffn_periodic", lib.pop_decode_ffn_periodic(
        _ptr(x), batch, d, _ptr(W_gate), _ptr(W_up), _ptr(W_downT), d_ff, _dtype(W_gate),
        _ptr(R), R.numel(), _ptr(C), C.numel(), float(r), int(step), int(period), _ptr(state.memory),
        _ptr(state.positions), _ptr(state.selected), _ptr(state.rows), _ptr(y), _ptr(ws), ws.numel(),
        _stream(stream)))
    return y


def pop_decode_topk_count(d_ff: int, r: float, n_R: int, n_C: int) -> int:
    """k, the candidates one decode step selects (the library's count)."""
    k = _c_i32()
    _check("pop_decode_topk_count", lib.pop_decode_topk_count(int(d_ff), float(r), int(n_R), int(n_C), ctypes.byref(k)))
    return int(k.value)


def pop_dense_ffn_decode(x, W_gate, W_up, W_downT, *, y=None, ws=None, stream=None):
    _dev(x, W_gate, W_up, W_downT)
    batch, d = x.shape
    d_ff = W_gate.shape[0]
    dev = W_gate.device
    if y is None:
        y = torch.empty((batch, d), dtype=torch.float32, device=dev)
    if ws is None:
        ws = workspace(pop_decode_workspace_bytes(batch, d, d_ff), dev)
    _check("pop_dense_ffn_decode", lib.pop_dense_ffn_decode(
        _ptr(x), batch, d, _ptr(W_gate), _ptr(W_up), _ptr(W_downT), d_ff, _dtype(W_gate),
        _ptr(y), _ptr(ws), ws.numel(), _stream(stream)))
    return y


def pop_dense_ffn_prefill_workspace_bytes(n_tokens: int, d: int, d_ff: int, dtype: str) -> int:
    return int(lib.pop_dense_ffn_prefill_workspace_bytes(n_tokens, d, d_ff, POP_BF16 if dtype == "bf16" else POP_F32))


def pop_dense_ffn_prefill(X, W_gate, W_up, W_downT, *, Y=None, ws=None, stream=None):
    """Y [n_tokens, d] (fp32): the dense gated MLP over the prompt tokens."""
    _dev(X, W_gate, W_up, W_downT)
    n_tokens, d = X.shape
    d_ff = W_gate.shape[0]
    dev = W_gate.device
    if Y is None:
        Y = torch.empty((n_tokens, d), dtype=torch.float32, device=dev)
    if ws is None:
        dt = "bf16" if W_gate.dtype == torch.bfloat16 else "f32"
        ws = workspace(max(pop_dense_ffn_prefill_workspace_bytes(n_tokens, d, d_ff, dt), 256), dev)
    _check("pop_dense_ffn_prefill", lib.pop_dense_ffn_prefill(
        _ptr(X), n_tokens, d, _ptr(W_gate), _ptr(W_up), _ptr(W_downT), d_ff, _dtype(W_gate),
        _ptr(Y), _ptr(ws), ws.numel(), _stream(stream)))
    return Y


# ---------------------------------------------------------------- mixture of experts
def pop_prefill_ffn_partition_workspace_bytes(n_tokens: int, d: int, d_ff: int, dtype: str) -> int:
    return int(lib.pop_prefill_ffn_partition_workspace_bytes(n_tokens, d, d_ff,
                                                             POP_BF16 if dtype == "bf16" else POP_F32))


def pop_prefill_ffn_partition(X, W_gate, W_up, W_downT, r: float, gamma: float, *, importance: bool = False,
                              Y=None, out=None, ws=None, stream=None):
    """(Y, R, C, P[, I]): the dense prompt FFN and the partition in one call, the
    importance taken inside the gate/up pass."""
    _dev(X, W_gate, W_up, W_downT)
    n_tokens, d = X.shape
    d_ff = W_gate.shape[0]
    dev = W_gate.device
    c = pop_partition_counts(d_ff, r, gamma)
    if Y is None:
        Y = torch.empty((n_tokens, d), dtype=torch.float32, device=dev)
    if out is None:
        R = torch.empty(c["n_R"], dtype=torch.int32, device=dev)
        C = torch.empty(c["n_C"], dtype=torch.int32, device=dev)
        P = torch.empty(c["n_P"], dtype=torch.int32, device=dev)
        I = torch.empty(d_ff, dtype=torch.float32, device=dev) if importance else None
    else:
        R, C, P, I = out
    if ws is None:
        dt = "bf16" if W_gate.dtype == torch.bfloat16 else "f32"
        ws = workspace(pop_prefill_ffn_partition_workspace_bytes(n_tokens, d, d_ff, dt), dev)
    _check("pop_prefill_ffn_partition", lib.pop_prefill_ffn_partition(
        _ptr(X), n_tokens, d, _ptr(W_gate), _ptr(W_up), _ptr(W_downT), d_ff, _dtype(W_gate), float(r),
        float(gamma), _ptr(Y), _ptr(R), _ptr(C), _ptr(P), _ptr(I), _ptr(ws), ws.numel(), _stream(stream)))
    return (Y, R, C, P, I) if importance else (Y, R, C, P)


def pop_moe_route_top2(logits, *, stream=None):
    """(experts [T, 2], weights [T, 2], offsets [E + 1], tokens [2T], slots [T, 2])."""
    _dev(logits)
    T, E = logits.shape
    dev = logits.device
    ex = torch.empty((T, 2), dtype=torch.int32, device=dev)
    wt = torch.empty((T, 2), dtype=torch.float32, device=dev)
    off = torch.empty(E + 1, dtype=torch.int32, device=dev)
    tok = torch.empty(2 * T, dtype=torch.int32, device=dev)
    slot = torch.empty((T, 2), dtype=torch.int32, device=dev)
    _check("pop_moe_route_top2", lib.pop_moe_route_top2(
        _ptr(logits), T, E, _ptr(ex), _ptr(wt), _ptr(off), _ptr(tok), _ptr(slot), _stream(stream)))
    return ex, wt, off, tok, slot


def pop_moe_prefill_partition(X, logits, W_up, r: float, gamma: float, *, importance: bool = False, out=None,
                              ws=None, stream=None):
    """(R [E, n_R], C [E, n_C], P [E, n_P][, I [E, d_ff]]) for stacked W_up [E, d_ff, d]."""
    _dev(X, logits, W_up)
    n_tokens, d = X.shape
    E, d_ff, _ = W_up.shape
    c = pop_partition_counts(d_ff, r, gamma)
    dev = W_up.device
    if out is None:
        R, C, P = (torch.empty((E, c[n]), dtype=torch.int32, device=dev) for n in ("n_R", "n_C", "n_P"))
        I = torch.empty((E, d_ff), dtype=torch.float32, device=dev) if importance else None
    else:
        R, C, P, I = out
    if ws is None:
        ws = workspace(lib.pop_moe_prefill_workspace_bytes(n_tokens, d, d_ff, E), dev)
    _check("pop_moe_prefill_partition", lib.pop_moe_prefill_partition(
        _ptr(X), n_tokens, d, _ptr(logits), E, _ptr(W_up), d_ff, _dtype(W_up), float(r), float(gamma),
        _ptr(R), _ptr(C), _ptr(P), _ptr(I), _ptr(ws), ws.numel(), _stream(stream)))
    return (R, C, P, I) if importance else (R, C, P)


def pop_moe_decode_workspace_bytes(n_tokens: int, d: int, d_ff: int, n_experts: int) -> int:
    return int(lib.pop_moe_decode_workspace_bytes(n_tokens, d, d_ff, n_experts))


def pop_moe_decode_ffn(x, logits, W_gate, W_up, W_downT, R, C, r: float, *, y=None, selected: bool = False,
                       ws=None, stream=None):
    """y [T, d] (fp32) for one MoE decode step; optionally the selected
    candidates [E, k] (rows of experts that received no token are left as they
    were: zero-initialised here)."""
    _dev(x, logits, W_gate, W_up, W_downT, R, C)
    T, d = x.shape
    E, d_ff, _ = W_gate.shape
    dev = W_gate.device
    if y is None:
        y = torch.empty((T, d), dtype=torch.float32, device=dev)
    S = None
    if selected:
        S = torch.zeros((E, pop_decode_topk_count(d_ff, r, R.shape[1], C.shape[1])), dtype=torch.int32, device=dev)
    if ws is None:
        ws = workspace(pop_moe_decode_workspace_bytes(T, d, d_ff, E), dev)
    _check("pop_moe_decode_ffn", lib.pop_moe_decode_ffn(
        _ptr(x), T, d, _ptr(logits), E, _ptr(W_gate), _ptr(W_up), _ptr(W_downT), d_ff, _dtype(W_gate),
        _ptr(R), R.shape[1], _ptr(C), C.shape[1], float(r), _ptr(y), _ptr(S), _ptr(ws), ws.numel(),
        _stream(stream)))
    return (y, S) if selected else y


# ---------------------------------------------------------------- stages
def pop_prefill_importance(X, W_up, *, out=None, ws=None, stream=None):
    """I [d_ff] (fp32): the importance of every channel from the prompt X."""
    _dev(X, W_up)
    n_tokens, d = X.shape
    d_ff = W_up.shape[0]
    I = torch.empty(d_ff, dtype=torch.float32, device=W_up.device) if out is None else out
    if ws is None:
        ws = workspace(lib.pop_prefill_importance_workspace_bytes(n_tokens, d, d_ff), W_up.device)
    _check("pop_prefill_importance", lib.pop_prefill_importance(
        _ptr(X), n_tokens, d, _ptr(W_up), d_ff, _dtype(W_up), _ptr(I), _ptr(ws), ws.numel(), _stream(stream)))
    return I


def pop_partition_select(I, r: float, gamma: float, *, out=None, stream=None):
    """(R, C, P) from an importance vector."""
    _dev(I)
    d_ff = I.numel()
    c = pop_partition_counts(d_ff, r, gamma)
    if out is None:
        out = tuple(torch.empty(c[n], dtype=torch.int32, device=I.device) for n in ("n_R", "n_C", "n_P"))
    R, C, P = out
    _check("pop_partition_select", lib.pop_partition_select(
        _ptr(I), d_ff, float(r), float(gamma), _ptr(R), _ptr(C), _ptr(P), _stream(stream)))
    return R, C, P


def pop_decode_gateup(x, W_gate, W_up, R, C, *, n_R=None, z=None, score=None, want_score=True, stream=None):
    """(z [batch, n_R + n_C], score [n_C]).  R=None with n_R given: identity rows."""
    _dev(x, W_gate, W_up, R, C)
    batch, d = x.shape
    d_ff = W_gate.shape[0]
    nR = R.numel() if R is not None else int(n_R)
    nC = C.numel() if C is not None else 0
    dev = W_gate.device
    if z is None:
        z = torch.empty((batch, nR + nC), dtype=torch.float32, device=dev)
    if score is None and want_score:
        score = torch.empty(nC, dtype=torch.float32, device=dev)
    _check("pop_decode_gateup", lib.pop_decode_gateup(
        _ptr(x), batch, d, _ptr(W_gate), _ptr(W_up), d_ff, _dtype(W_gate), _ptr(R), nR, _ptr(C), nC,
        _ptr(z), _ptr(score), _stream(stream)))
    return z, score


def pop_decode_select(score, C, k: int, *, positions=None, selected=None, stream=None):
    """(positions [k], selected [k]) of the k best candidates."""
    _dev(score, C)
    n_C = score.numel()
    dev = score.device
    if positions is None:
        positions = torch.empty(int(k), dtype=torch.int32, device=dev)
    if selected is None:
        selected = torch.empty(int(k), dtype=torch.int32, device=dev)
    _check("pop_decode_select", lib.pop_decode_select(
        _ptr(score), n_C, _ptr(C), int(k), _ptr(positions), _ptr(selected), _stream(stream)))
    return positions, selected


def pop_decode_down(z, W_downT, R, selected, positions, *, n_R=None, y=None, ws=None, stream=None):
    """y [batch, d] from z over R and the selected candidates."""
    _dev(z, W_downT, R, selected, positions)
    batch, n_A = z.shape
    d_ff, d = W_downT.shape
    nR = R.numel() if R is not None else int(n_R)
    k = positions.numel() if positions is not None else 0
    dev = W_downT.device
    if y is None:
        y = torch.empty((batch, d), dtype=torch.float32, device=dev)
    if ws is None:
        ws = workspace(lib.pop_decode_down_workspace_bytes(batch, d, nR + k), dev)
    _check("pop_decode_down", lib.pop_decode_down(
        _ptr(z), batch, n_A, _ptr(W_downT), d, d_ff, _dtype(W_downT), _ptr(R), nR, _ptr(selected), _ptr(positions), k,
        _ptr(y), _ptr(ws), ws.numel(), _stream(stream)))
    return y


# ---------------------------------------------------------------- kernel tracing
class Tracer:
    """Arms libpop's kernel tracing with raw HIP events (created through the HIP
    runtime) and reads the per-kernel elapsed times back.

        with Tracer(n) as tr:
            ... libpop calls ...
        torch.cuda.synchronize(); tr.intervals_ms()
    """

    # hipEventDisableSystemFence: the event's record skips the system-scope
    # release (a cache writeback between every two kernels otherwise).
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, n_events: int, flags: int = 0):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(_c_vp), ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), _c_vp, _c_vp]
        self.hip.hipEventDestroy.argtypes = [_c_vp]
        self.n = int(n_events)
        self.events = (_c_vp * self.n)()
        for i in range(self.n):
            h = _c_vp()
            if self.hip.hipEventCreateWithFlags(ctypes.byref(h), ctypes.c_uint(flags)) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            self.events[i] = h
        self.used = 0

    def __enter__(self):
        _check("pop_set_trace_events", lib.pop_set_trace_events(self.events, self.n))
        return self

    def __exit__(self, *exc):
        self.used = int(lib.pop_trace_recorded())
        lib.pop_set_trace_events(None, 0)
        return False

    def elapsed_ms(self, i: int, j: int) -> float:
        out = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(out), self.events[i], self.events[j]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(out.value)

    def close(self):
        for i in range(self.n):
            self.hip.hipEventDestroy(self.events[i])
        self.n = 0


# ---------------------------------------------------------------- decoder layer
class Layer:
    """One decoder layer's shape, weights and dtype for the pop_layer_* calls.

    weights: dict of device tensors attn_norm [d] (fp32), Wqkv_T [d, (H + 2 H_kv) hd],
    Wo_T [H hd, d], ffn_norm [d] (fp32), W_gate, W_up, W_downT [d_ff, d] (all in one
    dtype).  The tensors must outlive every call made with this object."""

    def __init__(self, d: int, n_heads: int, n_kv_heads: int, head_dim: int, d_ff: int, cache_len: int,
                 weights: dict, eps: float = 1e-5, rope_theta: float = 10000.0):
        self.shape = LayerShape(d, n_heads, n_kv_heads, head_dim, d_ff, cache_len, eps, rope_theta)
        _dev(*weights.values())
        self.weights = dict(weights)
        self.ptrs = LayerWeights(*[weights[n].data_ptr() for n, _ in LayerWeights._fields_])
        self.dt = _dtype(weights["W_gate"])

    def cache(self, batch: int, device=None):
        """Zeroed (K, V) caches [batch, H_kv, cache_len, hd] in the weights' dtype."""
        s = self.shape
        shp = (batch, s.n_kv_heads, s.cache_len, s.head_dim)
        dtype = self.weights["W_gate"].dtype
        dev = device or self.weights["W_gate"].device
        return torch.zeros(shp, dtype=dtype, device=dev), torch.zeros(shp, dtype=dtype, device=dev)


def pop_layer_prefill_workspace_bytes(batch: int, n_tokens: int, layer: Layer) -> int:
    return int(lib.pop_layer_prefill_workspace_bytes(int(batch), int(n_tokens), ctypes.byref(layer.shape), layer.dt))


def pop_layer_decode_workspace_bytes(batch: int, layer: Layer) -> int:
    return int(lib.pop_layer_decode_workspace_bytes(int(batch), ctypes.byref(layer.shape), layer.dt))


def pop_layer_prefill(x, layer: Layer, K, V, r: float, gamma: float, *, importance: bool = False, out=None,
                      ws=None, stream=None):
    """The prompt's pass: x [batch, n_tokens, d] (fp32) is updated in place; the
    caches get positions 0 .. n_tokens - 1.  Returns (R, C, P[, I])."""
    _dev(x, K, V)
    batch, n_tokens, d = x.shape
    d_ff = layer.shape.d_ff
    c = pop_partition_counts(d_ff, r, gamma)
    dev = x.device
    if out is None:
        R = torch.empty(c["n_R"], dtype=torch.int32, device=dev)
        C = torch.empty(c["n_C"], dtype=torch.int32, device=dev)
        P = torch.empty(c["n_P"], dtype=torch.int32, device=dev)
        I = torch.empty(d_ff, dtype=torch.float32, device=dev) if importance else None
    else:
        R, C, P, I = out
    if ws is None:
        ws = workspace(pop_layer_prefill_workspace_bytes(batch, n_tokens, layer), dev)
    _check("pop_layer_prefill", lib.pop_layer_prefill(
        _ptr(x), batch, n_tokens, ctypes.byref(layer.shape), ctypes.byref(layer.ptrs), layer.dt, _ptr(K), _ptr(V),
        float(r), float(gamma), _ptr(R), _ptr(C), _ptr(P), _ptr(I), _ptr(ws), ws.numel(), _stream(stream)))
    return (R, C, P, I) if importance else (R, C, P)


def pop_layer_decode(x, layer: Layer, K, V, pos, R, C, r: float, *, dense_ffn: bool = False, selected=None,
                     ws=None, stream=None):
    """One decode step: x [batch, d] (fp32) is updated in place; pos is a device
    int32 tensor [1] holding the token's position.  ``selected`` (optional,
    int32 [k]) receives the chosen candidates.  Returns x."""
    _dev(x, K, V, pos, R, C, selected)
    batch = x.shape[0]
    if ws is None:
        ws = workspace(pop_layer_decode_workspace_bytes(batch, layer), x.device)
    nR = 0 if R is None else R.numel()
    nC = 0 if C is None else C.numel()
    _check("pop_layer_decode", lib.pop_layer_decode(
        _ptr(x), batch, ctypes.byref(layer.shape), ctypes.byref(layer.ptrs), layer.dt, _ptr(K), _ptr(V), _ptr(pos),
        _ptr(R), nR, _ptr(C), nC, float(r), int(bool(dense_ffn)), _ptr(selected), _ptr(ws), ws.numel(),
        _stream(stream)))
    return x


def pop_hbm_read_probe(src, sink, blocks: int = 1024, *, stream=None):
    """Reads src (a device tensor) once; sink: device int32/uint32 [blocks * 256]."""
    _dev(src, sink)
    _check("pop_hbm_read_probe", lib.pop_hbm_read_probe(_ptr(src), src.numel() * src.element_size(), _ptr(sink),
                                                        int(blocks), _stream(stream)))
