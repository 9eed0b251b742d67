"""The whole routing path on device buffers: route -> greedy replica
assignment -> layout -> dispatch -> expert stand-in -> combine, each step one
call into the HIP library. Torch provides the device memory and the stream.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import binding as B


@dataclass
class Buffers:
    p: B.Problem
    logits: torch.Tensor
    x: torch.Tensor
    rep: torch.Tensor | None
    maxrep: int
    ws: torch.Tensor
    idx: torch.Tensor
    w: torch.Tensor
    counts: torch.Tensor
    assign: torch.Tensor
    active: torch.Tensor
    rank_of: torch.Tensor
    expert_offsets: torch.Tensor
    rank_offsets: torch.Tensor
    pos: torch.Tensor
    src: torch.Tensor
    dedup: torch.Tensor
    send: torch.Tensor
    y: torch.Tensor
    out: torch.Tensor


def allocate(p: B.Problem, logits: torch.Tensor, x: torch.Tensor, rep: torch.Tensor | None = None,
             device: str | torch.device = "cuda") -> Buffers:
    """Device buffers for one batch. `logits` [T, E] f32 and `x` [T, H] in the
    activation dtype are copied to the device; `rep` is an int32 [E, maxrep]
    replica table or None."""
    dev = torch.device(device)
    T, E, k, H, R = p.T, p.E, p.k, p.H, p.R
    act = B._TORCH_ACT[p.act_dtype]
    i32 = dict(dtype=torch.int32, device=dev)
    out_dt = torch.float32 if p.flags & B.MOE_FLAG_OUT_F32 else act
    rep_d = None if rep is None else rep.to(dev, torch.int32).contiguous()
    maxrep = 1 if rep is None else int(rep.shape[1])
    ws_bytes = B.moe_workspace_bytes(p)
    return Buffers(
        p=p, logits=logits.to(dev, torch.float32).contiguous(), x=x.to(dev).contiguous(),
        rep=rep_d, maxrep=maxrep,
        ws=torch.empty(ws_bytes, dtype=torch.uint8, device=dev),
        idx=torch.empty(T * k, **i32), w=torch.empty(T * k, dtype=torch.float32, device=dev),
        counts=torch.empty(E, **i32), assign=torch.empty(E, **i32), active=torch.empty(R, **i32),
        rank_of=torch.empty(E, **i32), expert_offsets=torch.empty(E, **i32),
        rank_offsets=torch.empty(R + 1, **i32), pos=torch.empty(T * k, **i32),
        src=torch.empty(T * k, **i32), dedup=torch.empty(R, **i32),
        send=torch.empty(T * k, H, dtype=act, device=dev),
        y=torch.empty(T * k, H, dtype=act, device=dev),
        out=torch.empty(T, H, dtype=out_dt, device=dev))


def route(b: Buffers, stream=None) -> None:
    B.moe_route(b.p, b.logits, b.idx, b.w, b.counts, b.ws, stream)


def assign(b: Buffers, stream=None) -> None:
    B.moe_assign_replicas(b.p, b.counts, b.rep, b.maxrep, b.assign, b.active, stream)


def layout(b: Buffers, stream=None) -> None:
    B.moe_layout(b.p, b.idx, b.assign, b.rep, b.maxrep, b.rank_of, b.expert_offsets,
                 b.rank_offsets, b.pos, b.src, b.dedup, b.ws, stream)


def route_assign_layout(b: Buffers, stream=None) -> None:
    """route, assign and layout in one library call (two launches for a
    decode-sized batch)."""
    B.moe_route_assign_layout(b.p, b.logits, b.rep, b.maxrep, b.idx, b.w, b.counts, b.assign,
                              b.active, b.rank_of, b.expert_offsets, b.rank_offsets, b.pos, b.src,
                              b.dedup, b.ws, stream)


def dispatch(b: Buffers, stream=None) -> None:
    B.moe_dispatch(b.p, b.x, b.pos, b.send, stream)


def standin(b: Buffers, stream=None) -> None:
    B.moe_expert_standin(b.p, b.send, b.src, b.idx, b.y, stream)


def combine(b: Buffers, stream=None) -> None:
    B.moe_combine(b.p, b.y, b.pos, b.w, b.out, stream)


STEPS = (route, assign, layout, dispatch, standin, combine)
# the same pass with route, assign and layout in one call
FUSED_STEPS = (route_assign_layout, dispatch, standin, combine)


def run(b: Buffers, stream=None) -> None:
    for step in STEPS:
        step(b, stream)


def capture(b: Buffers, steps=STEPS) -> torch.cuda.CUDAGraph:
    """Records one pass of `steps` (the whole path by default) into a HIP
    graph. The library only enqueues kernels (no memset, allocation or
    synchronisation), so the pass replays with one launch; the buffers of `b`
    are the graph's inputs and outputs: copy a new batch into b.logits / b.x
    in place, then replay. One eager pass on a side stream comes first, as
    torch asks before a capture."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for step in steps:
            step(b)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for step in steps:
            step(b)
    return g


def record(b: Buffers, ss: SingleSend | None = None) -> dict:
    """Host-side record of one routed batch: what "METRO AllGather vs AllToAll
    for MoE decode", section "Distinguish METRO from backend names", asks to
    keep beside collective traces (buffer sizes per destination rank and the
    expert replica chosen for each expert's global count), plus the dedup
    total and the activated experts per GPU. Reads back 2E + 3R + 1 ints of
    metadata (R + 1 more with `ss`; this synchronises the stream), never the
    rows.

    send_bytes[r] is rank r's segment of the send buffer, the size of the
    all-to-all chunk for destination r; with `ss`, ss_send_bytes[r] is the
    same for the single-send buffer."""
    p = b.p
    row_bytes = p.H * 2  # 16-bit activations
    roff = b.rank_offsets.cpu().tolist()
    rec = {
        "T": p.T, "E": p.E, "k": p.k, "H": p.H, "R": p.R,
        "send_bytes": [(roff[r + 1] - roff[r]) * row_bytes for r in range(p.R)],
        "rows": roff[-1],
        "dedup_rows": int(b.dedup.sum().item()),
        "active_per_gpu": b.active.cpu().tolist(),
        "counts": b.counts.cpu().tolist(),
        "assign": b.assign.cpu().tolist(),
    }
    if ss is not None:
        so = ss.ss_rank_offsets.cpu().tolist()
        rec["ss_send_bytes"] = [(so[r + 1] - so[r]) * row_bytes for r in range(p.R)]
    return rec


@dataclass
class SingleSend:
    """Single-send buffers: one row per (token, destination rank). The row
    capacity is T * min(k, R), the most distinct (token, rank) pairs a batch
    can have, so no count has to be read back before the dispatch."""
    ss_rank_offsets: torch.Tensor
    ss_row: torch.Tensor
    ss_token: torch.Tensor
    send_ss: torch.Tensor


def allocate_single_send(b: Buffers) -> SingleSend:
    p, dev = b.p, b.idx.device
    n, cap = p.T * p.k, p.T * min(p.k, p.R)
    i32 = dict(dtype=torch.int32, device=dev)
    return SingleSend(ss_rank_offsets=torch.empty(p.R + 1, **i32), ss_row=torch.empty(n, **i32),
                      ss_token=torch.empty(n, **i32),
                      send_ss=torch.empty(cap, p.H, dtype=b.send.dtype, device=dev))


def layout_single_send(b: Buffers, ss: SingleSend, stream=None) -> None:
    B.moe_layout_single_send(b.p, b.idx, b.assign, b.rep, b.maxrep, b.rank_of, b.expert_offsets,
                             b.rank_offsets, b.pos, b.src, b.dedup, ss.ss_rank_offsets, ss.ss_row,
                             ss.ss_token, b.ws, stream)


def route_assign_layout_single_send(b: Buffers, ss: SingleSend, stream=None) -> None:
    """route, assign and the single-send layout in one library call (three
    launches for a batch without a replica table)."""
    B.moe_route_assign_layout_single_send(b.p, b.logits, b.rep, b.maxrep, b.idx, b.w, b.counts,
                                          b.assign, b.active, b.rank_of, b.expert_offsets,
                                          b.rank_offsets, b.pos, b.src, b.dedup,
                                          ss.ss_rank_offsets, ss.ss_row, ss.ss_token, b.ws, stream)


def single_send_dispatch(b: Buffers, ss: SingleSend, stream=None) -> None:
    B.moe_single_send_dispatch(b.p, b.x, ss.ss_row, ss.send_ss, stream)


def single_send_expand(b: Buffers, ss: SingleSend, stream=None) -> None:
    """Fills b.send from the single-send rows (what dispatch writes)."""
    B.moe_single_send_expand(b.p, ss.send_ss, ss.ss_rank_offsets, ss.ss_token, ss.ss_row, b.pos,
                             b.send, stream)


@dataclass
class Stats:
    """Routing-statistics outputs: send_counts [R, R], coselect [E, E] (or
    None), stats [4] = max/mean, Gini, Dirichlet alpha, locality."""
    send_counts: torch.Tensor
    coselect: torch.Tensor | None
    stats: torch.Tensor


def allocate_stats(b: Buffers, coselect: bool = True) -> Stats:
    p, dev = b.p, b.idx.device
    return Stats(send_counts=torch.empty(p.R, p.R, dtype=torch.int32, device=dev),
                 coselect=torch.empty(p.E, p.E, dtype=torch.int32, device=dev) if coselect else None,
                 stats=torch.empty(4, dtype=torch.float64, device=dev))


def routing_stats(b: Buffers, st: Stats, stream=None) -> None:
    B.moe_routing_stats(b.p, b.idx, b.counts, b.rank_of, st.send_counts, st.coselect, st.stats,
                        stream)


@dataclass
class Split:
    """Token-balanced (EPLB-style) routing outputs: the GPU of each pair and,
    per GPU, the activated replicas and the pairs served."""
    gpu_of_pair: torch.Tensor
    active: torch.Tensor
    tokens: torch.Tensor


def allocate_split(b: Buffers) -> Split:
    p, dev = b.p, b.idx.device
    i32 = dict(dtype=torch.int32, device=dev)
    return Split(gpu_of_pair=torch.empty(p.T * p.k, **i32), active=torch.empty(p.R, **i32),
                 tokens=torch.empty(p.R, **i32))


def token_balanced_split(b: Buffers, sp: Split, stream=None) -> None:
    B.moe_token_balanced_split(b.p, b.idx, b.counts, b.pos, b.expert_offsets, b.rep, b.maxrep,
                               sp.gpu_of_pair, sp.active, sp.tokens, stream)
