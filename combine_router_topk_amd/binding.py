"""ctypes binding of libmoe_route.so: one Python function per C entry point,
same names, same argument order (see include/moe_route.h).

Only argument marshalling happens here: torch tensors (device memory) become
pointers, the stream becomes torch's current HIP stream unless given, and
tensor sizes are checked against the problem so the library can never be
handed a buffer shorter than the shape it is told about. Every step of the
routing path runs in the HIP library; there is no fallback. If the library is
missing, or was built from sources other than those beside it (its
moe_build_id() differs from the digest of csrc/ and include/), importing this
module raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

from . import build as _build

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_route.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_F16, MOE_BF16 = 1, 2
MOE_FLAG_GREEDY_ID_ORDER = 1 << 0
MOE_FLAG_OUT_F32 = 1 << 1
MOE_MAX_E, MOE_MAX_K, MOE_MAX_R, MOE_MAX_REP = 1024, 16, 1024, 16
MOE_MAX_ROWS = (1 << 24) - 1
MOE_NOALLOC_SCRATCH_BYTES = 2 << 20

EXPORTED = ("moe_version", "moe_build_id", "moe_status_string", "moe_last_error", "moe_workspace_bytes",
            "moe_route", "moe_assign_replicas", "moe_layout", "moe_route_assign_layout",
            "moe_route_assign_layout_noalloc", "moe_route_assign_layout_single_send",
            "moe_layout_single_send",
            "moe_single_send_dispatch", "moe_single_send_expand", "moe_dispatch",
            "moe_expert_standin", "moe_combine", "moe_combine_backward", "moe_dispatch_backward",
            "moe_routing_stats", "moe_token_balanced_split")

_TORCH_ACT = {MOE_F16: torch.float16, MOE_BF16: torch.bfloat16}


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({_status_string(status)}): {detail}")


class Problem(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("E", ctypes.c_int32), ("k", ctypes.c_int32),
                ("H", ctypes.c_int32), ("R", ctypes.c_int32), ("act_dtype", ctypes.c_int32),
                ("flags", ctypes.c_uint32)]

    def __repr__(self):
        return (f"Problem(T={self.T}, E={self.E}, k={self.k}, H={self.H}, R={self.R}, "
                f"act_dtype={self.act_dtype}, flags={self.flags})")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python combine_router_topk_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(Problem)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    sig = {
        "moe_version": (i32, []),
        "moe_build_id": (ctypes.c_char_p, []),
        "moe_status_string": (ctypes.c_char_p, [i32]),
        "moe_last_error": (ctypes.c_char_p, []),
        "moe_workspace_bytes": (i32, [P, ctypes.POINTER(sz)]),
        "moe_route": (i32, [P, vp, vp, vp, vp, vp, sz, vp]),
        "moe_assign_replicas": (i32, [P, vp, vp, i32, vp, vp, vp]),
        "moe_layout": (i32, [P, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "moe_route_assign_layout": (i32, [P, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                          vp, vp, sz, vp]),
        "moe_route_assign_layout_noalloc": (i32, [P, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp,
                                                  vp, vp, vp, vp]),
        "moe_route_assign_layout_single_send": (i32, [P, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp,
                                                      vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "moe_layout_single_send": (i32, [P, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                         vp, sz, vp]),
        "moe_single_send_dispatch": (i32, [P, vp, vp, vp, i32, vp]),
        "moe_single_send_expand": (i32, [P, vp, vp, vp, vp, vp, i32, vp, vp]),
        "moe_dispatch": (i32, [P, vp, vp, vp, vp]),
        "moe_expert_standin": (i32, [P, vp, vp, vp, vp, vp]),
        "moe_combine": (i32, [P, vp, vp, vp, vp, vp]),
        "moe_combine_backward": (i32, [P, vp, vp, vp, vp, vp, vp, vp]),
        "moe_dispatch_backward": (i32, [P, vp, vp, vp, vp]),
        "moe_routing_stats": (i32, [P, vp, vp, vp, vp, vp, vp, vp]),
        "moe_token_balanced_split": (i32, [P, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype, f.argtypes = res, args
    built, want = lib.moe_build_id().decode(), _build.source_digest()
    if built != want:
        raise ImportError(f"{LIB_PATH} was built from other sources (build id {built}, sources "
                          f"{want}); rebuild with `python combine_router_topk_amd/build.py`")
    return lib


_lib = _load()


def _status_string(status: int) -> str:
    return _lib.moe_status_string(status).decode()


def _check(status: int, where: str) -> None:
    if status != MOE_OK:
        raise MoeError(status, where, _lib.moe_last_error().decode())


def make_problem(T: int, E: int, k: int, H: int, R: int, act_dtype: int, flags: int = 0) -> Problem:
    return Problem(T, E, k, H, R, act_dtype, flags)


def _ptr(t: torch.Tensor | None, dtype: torch.dtype | None, numel: int | None, name: str):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name}: {t.numel()} elements, need {numel}")
    return ctypes.c_void_p(t.data_ptr())


def _nbytes(t: torch.Tensor | None) -> int:
    """Byte size of a workspace tensor; 0 for None (the library then reports
    the NULL pointer)."""
    return 0 if t is None else t.numel() * t.element_size()


def _rows(t: torch.Tensor | None) -> int:
    """Row count of a single-send buffer (its capacity); 0 for None."""
    return 0 if t is None else t.shape[0]


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def moe_version() -> int:
    return _lib.moe_version()


def moe_build_id() -> str:
    return _lib.moe_build_id().decode()


def moe_status_string(status: int) -> str:
    return _status_string(status)


def moe_last_error() -> str:
    return _lib.moe_last_error().decode()


def moe_workspace_bytes(p: Problem) -> int:
    n = ctypes.c_size_t(0)
    _check(_lib.moe_workspace_bytes(ctypes.byref(p), ctypes.byref(n)), "moe_workspace_bytes")
    return n.value


def moe_route(p: Problem, logits, idx, w, counts, ws, stream=None) -> None:
    n = p.T * p.k
    _check(_lib.moe_route(ctypes.byref(p),
                          _ptr(logits, torch.float32, p.T * p.E, "logits"),
                          _ptr(idx, torch.int32, n, "idx"), _ptr(w, torch.float32, n, "w"),
                          _ptr(counts, torch.int32, p.E, "counts"), _ptr(ws, None, None, "ws"),
                          _nbytes(ws), _stream(stream)), "moe_route")


def moe_assign_replicas(p: Problem, counts, rep, maxrep: int, assign, active, stream=None) -> None:
    _check(_lib.moe_assign_replicas(ctypes.byref(p), _ptr(counts, torch.int32, p.E, "counts"),
                                    _ptr(rep, torch.int32, p.E * maxrep if rep is not None else 0, "rep"),
                                    maxrep, _ptr(assign, torch.int32, p.E, "assign"),
                                    _ptr(active, torch.int32, p.R, "active"), _stream(stream)),
           "moe_assign_replicas")


def moe_layout(p: Problem, idx, assign, rep, maxrep: int, rank_of, expert_offsets, rank_offsets,
               pos, src, dedup, ws, stream=None) -> None:
    n = p.T * p.k
    _check(_lib.moe_layout(ctypes.byref(p), _ptr(idx, torch.int32, n, "idx"),
                           _ptr(assign, torch.int32, p.E, "assign"),
                           _ptr(rep, torch.int32, p.E * maxrep if rep is not None else 0, "rep"),
                           maxrep, _ptr(rank_of, torch.int32, p.E, "rank_of"),
                           _ptr(expert_offsets, torch.int32, p.E, "expert_offsets"),
                           _ptr(rank_offsets, torch.int32, p.R + 1, "rank_offsets"),
                           _ptr(pos, torch.int32, n, "pos"), _ptr(src, torch.int32, n, "src"),
                           _ptr(dedup, torch.int32, p.R, "dedup"), _ptr(ws, None, None, "ws"),
                           _nbytes(ws), _stream(stream)), "moe_layout")


def moe_route_assign_layout(p: Problem, logits, rep, maxrep: int, idx, w, counts, assign, active,
                            rank_of, expert_offsets, rank_offsets, pos, src, dedup, ws,
                            stream=None) -> None:
    n = p.T * p.k
    _check(_lib.moe_route_assign_layout(
        ctypes.byref(p), _ptr(logits, torch.float32, p.T * p.E, "logits"),
        _ptr(rep, torch.int32, p.E * maxrep if rep is not None else 0, "rep"), maxrep,
        _ptr(idx, torch.int32, n, "idx"), _ptr(w, torch.float32, n, "w"),
        _ptr(counts, torch.int32, p.E, "counts"), _ptr(assign, torch.int32, p.E, "assign"),
        _ptr(active, torch.int32, p.R, "active"), _ptr(rank_of, torch.int32, p.E, "rank_of"),
        _ptr(expert_offsets, torch.int32, p.E, "expert_offsets"),
        _ptr(rank_offsets, torch.int32, p.R + 1, "rank_offsets"),
        _ptr(pos, torch.int32, n, "pos"), _ptr(src, torch.int32, n, "src"),
        _ptr(dedup, torch.int32, p.R, "dedup"), _ptr(ws, None, None, "ws"), _nbytes(ws),
        _stream(stream)), "moe_route_assign_layout")


def moe_route_assign_layout_single_send(p: Problem, logits, rep, maxrep: int, idx, w, counts,
                                        assign, active, rank_of, expert_offsets, rank_offsets,
                                        pos, src, dedup, ss_rank_offsets, ss_row, ss_token, ws,
                                        stream=None) -> None:
    n = p.T * p.k
    _check(_lib.moe_route_assign_layout_single_send(
        ctypes.byref(p), _ptr(logits, torch.float32, p.T * p.E, "logits"),
        _ptr(rep, torch.int32, p.E * maxrep if rep is not None else 0, "rep"), maxrep,
        _ptr(idx, torch.int32, n, "idx"), _ptr(w, torch.float32, n, "w"),
        _ptr(counts, torch.int32, p.E, "counts"), _ptr(assign, torch.int32, p.E, "assign"),
        _ptr(active, torch.int32, p.R, "active"), _ptr(rank_of, torch.int32, p.E, "rank_of"),
        _ptr(expert_offsets, torch.int32, p.E, "expert_offsets"),
        _ptr(rank_offsets, torch.int32, p.R + 1, "rank_offsets"),
        _ptr(pos, torch.int32, n, "pos"), _ptr(src, torch.int32, n, "src"),
        _ptr(dedup, torch.int32, p.R, "dedup"),
        _ptr(ss_rank_offsets, torch.int32, p.R + 1, "ss_rank_offsets"),
        _ptr(ss_row, torch.int32, n, "ss_row"), _ptr(ss_token, torch.int32, n, "ss_token"),
        _ptr(ws, None, None, "ws"), _nbytes(ws), _stream(stream)),
        "moe_route_assign_layout_single_send")


def moe_route_assign_layout_noalloc(p: Problem, logits, rep, maxrep: int, idx, w, counts, assign,
                                    active, rank_of, expert_offsets, rank_offsets, pos, src, dedup,
                                    stream=None) -> None:
    n = p.T * p.k
    _check(_lib.moe_route_assign_layout_noalloc(
        ctypes.byref(p), _ptr(logits, torch.float32, p.T * p.E, "logits"),
        _ptr(rep, torch.int32, p.E * maxrep if rep is not None else 0, "rep"), maxrep,
        _ptr(idx, torch.int32, n, "idx"), _ptr(w, torch.float32, n, "w"),
        _ptr(counts, torch.int32, p.E, "counts"), _ptr(assign, torch.int32, p.E, "assign"),
        _ptr(active, torch.int32, p.R, "active"), _ptr(rank_of, torch.int32, p.E, "rank_of"),
        _ptr(expert_offsets, torch.int32, p.E, "expert_offsets"),
        _ptr(rank_offsets, torch.int32, p.R + 1, "rank_offsets"),
        _ptr(pos, torch.int32, n, "pos"), _ptr(src, torch.int32, n, "src"),
        _ptr(dedup, torch.int32, p.R, "dedup"), _stream(stream)),
        "moe_route_assign_layout_noalloc")


def moe_layout_single_send(p: Problem, idx, assign, rep, maxrep: int, rank_of, expert_offsets,
                           rank_offsets, pos, src, dedup, ss_rank_offsets, ss_row, ss_token, ws,
                           stream=None) -> None:
    n = p.T * p.k
    _check(_lib.moe_layout_single_send(
        ctypes.byref(p), _ptr(idx, torch.int32, n, "idx"), _ptr(assign, torch.int32, p.E, "assign"),
        _ptr(rep, torch.int32, p.E * maxrep if rep is not None else 0, "rep"), maxrep,
        _ptr(rank_of, torch.int32, p.E, "rank_of"),
        _ptr(expert_offsets, torch.int32, p.E, "expert_offsets"),
        _ptr(rank_offsets, torch.int32, p.R + 1, "rank_offsets"),
        _ptr(pos, torch.int32, n, "pos"), _ptr(src, torch.int32, n, "src"),
        _ptr(dedup, torch.int32, p.R, "dedup"),
        _ptr(ss_rank_offsets, torch.int32, p.R + 1, "ss_rank_offsets"),
        _ptr(ss_row, torch.int32, n, "ss_row"), _ptr(ss_token, torch.int32, n, "ss_token"),
        _ptr(ws, None, None, "ws"), _nbytes(ws), _stream(stream)),
        "moe_layout_single_send")


def moe_single_send_dispatch(p: Problem, x, ss_row, send_ss, stream=None) -> None:
    """send_ss holds the single-send rows; its row count is the capacity."""
    act = _TORCH_ACT.get(p.act_dtype)
    cap = _rows(send_ss)
    _check(_lib.moe_single_send_dispatch(ctypes.byref(p), _ptr(x, act, p.T * p.H, "x"),
                                         _ptr(ss_row, torch.int32, p.T * p.k, "ss_row"),
                                         _ptr(send_ss, act, cap * p.H, "send_ss"), cap,
                                         _stream(stream)), "moe_single_send_dispatch")


def moe_single_send_expand(p: Problem, send_ss, ss_rank_offsets, ss_token, ss_row, pos, send,
                           stream=None) -> None:
    """send_ss holds the single-send rows; its row count is the capacity."""
    act = _TORCH_ACT.get(p.act_dtype)
    n = p.T * p.k
    cap = _rows(send_ss)
    _check(_lib.moe_single_send_expand(ctypes.byref(p), _ptr(send_ss, act, cap * p.H, "send_ss"),
                                       _ptr(ss_rank_offsets, torch.int32, p.R + 1, "ss_rank_offsets"),
                                       _ptr(ss_token, torch.int32, min(cap, n), "ss_token"),
                                       _ptr(ss_row, torch.int32, n, "ss_row"),
                                       _ptr(pos, torch.int32, n, "pos"), cap,
                                       _ptr(send, act, n * p.H, "send"), _stream(stream)),
           "moe_single_send_expand")


def moe_dispatch(p: Problem, x, pos, send, stream=None) -> None:
    act = _TORCH_ACT.get(p.act_dtype)
    _check(_lib.moe_dispatch(ctypes.byref(p), _ptr(x, act, p.T * p.H, "x"),
                             _ptr(pos, torch.int32, p.T * p.k, "pos"),
                             _ptr(send, act, p.T * p.k * p.H, "send"), _stream(stream)),
           "moe_dispatch")


def moe_expert_standin(p: Problem, send, src, idx, y, stream=None) -> None:
    act = _TORCH_ACT.get(p.act_dtype)
    n = p.T * p.k
    _check(_lib.moe_expert_standin(ctypes.byref(p), _ptr(send, act, n * p.H, "send"),
                                   _ptr(src, torch.int32, n, "src"), _ptr(idx, torch.int32, n, "idx"),
                                   _ptr(y, act, n * p.H, "y"), _stream(stream)),
           "moe_expert_standin")


def moe_combine(p: Problem, y, pos, w, out, stream=None) -> None:
    act = _TORCH_ACT.get(p.act_dtype)
    out_dt = torch.float32 if p.flags & MOE_FLAG_OUT_F32 else act
    n = p.T * p.k
    _check(_lib.moe_combine(ctypes.byref(p), _ptr(y, act, n * p.H, "y"),
                            _ptr(pos, torch.int32, n, "pos"), _ptr(w, torch.float32, n, "w"),
                            _ptr(out, out_dt, p.T * p.H, "out"), _stream(stream)), "moe_combine")


def moe_combine_backward(p: Problem, dout, y, pos, w, dy, dw, stream=None) -> None:
    """dy and/or dw (either may be None); y may be None without dw and w
    without dy."""
    act = _TORCH_ACT.get(p.act_dtype)
    n = p.T * p.k
    _check(_lib.moe_combine_backward(ctypes.byref(p), _ptr(dout, act, p.T * p.H, "dout"),
                                     _ptr(y, act, n * p.H, "y"), _ptr(pos, torch.int32, n, "pos"),
                                     _ptr(w, torch.float32, n, "w"), _ptr(dy, act, n * p.H, "dy"),
                                     _ptr(dw, torch.float32, n, "dw"), _stream(stream)),
           "moe_combine_backward")


def moe_dispatch_backward(p: Problem, dsend, pos, dx, stream=None) -> None:
    act = _TORCH_ACT.get(p.act_dtype)
    out_dt = torch.float32 if p.flags & MOE_FLAG_OUT_F32 else act
    n = p.T * p.k
    _check(_lib.moe_dispatch_backward(ctypes.byref(p), _ptr(dsend, act, n * p.H, "dsend"),
                                      _ptr(pos, torch.int32, n, "pos"),
                                      _ptr(dx, out_dt, p.T * p.H, "dx"), _stream(stream)),
           "moe_dispatch_backward")


def moe_routing_stats(p: Problem, idx, counts, rank_of, send_counts, coselect, stats,
                      stream=None) -> None:
    """coselect may be None; stats is a float64 tensor of 4."""
    _check(_lib.moe_routing_stats(ctypes.byref(p), _ptr(idx, torch.int32, p.T * p.k, "idx"),
                                  _ptr(counts, torch.int32, p.E, "counts"),
                                  _ptr(rank_of, torch.int32, p.E, "rank_of"),
                                  _ptr(send_counts, torch.int32, p.R * p.R, "send_counts"),
                                  _ptr(coselect, torch.int32, p.E * p.E, "coselect"),
                                  _ptr(stats, torch.float64, 4, "stats"), _stream(stream)),
           "moe_routing_stats")


def moe_token_balanced_split(p: Problem, idx, counts, pos, expert_offsets, rep, maxrep: int,
                             gpu_of_pair, active, tokens, stream=None) -> None:
    n = p.T * p.k
    _check(_lib.moe_token_balanced_split(
        ctypes.byref(p), _ptr(idx, torch.int32, n, "idx"), _ptr(counts, torch.int32, p.E, "counts"),
        _ptr(pos, torch.int32, n, "pos"), _ptr(expert_offsets, torch.int32, p.E, "expert_offsets"),
        _ptr(rep, torch.int32, p.E * maxrep if rep is not None else 0, "rep"), maxrep,
        _ptr(gpu_of_pair, torch.int32, n, "gpu_of_pair"), _ptr(active, torch.int32, p.R, "active"),
        _ptr(tokens, torch.int32, p.R, "tokens"), _stream(stream)), "moe_token_balanced_split")
