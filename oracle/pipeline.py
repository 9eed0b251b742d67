"""The whole routing path in the order the METRO page gives it (top-k, demand
vector, replica choice), followed by the dispatch layout, the dispatch, the
expert stand-in and the combine (oracle).

Source: "METRO AllGather vs AllToAll for MoE decode", section "METRO AllGather
vs AllToAll changes the routing information".
"""
from __future__ import annotations

import numpy as np

from .layout import dedup_counts, expert_ranks, permutation, segment_offsets
from .replicas import greedy_assign
from .route import demand_vector, gate_weights, topk_select
from .rows import combine, dispatch_rows, expert_standin


def route_and_layout(T: int, E: int, k: int, R: int, logits: np.ndarray,
                     rep: np.ndarray | None = None, order: str = "constrained") -> dict:
    """All index outputs of the path for one batch (they are small at every
    workload size)."""
    assert logits.shape == (T, E)
    idx = topk_select(logits, k)
    w = gate_weights(logits, idx)
    counts = demand_vector(idx, E)
    assign, active = greedy_assign(counts, R, rep, order)
    rank_of = expert_ranks(E, R, rep, assign)
    expert_offsets, rank_offsets = segment_offsets(counts, rank_of, R)
    pos, src = permutation(idx, rank_of)
    dedup = dedup_counts(idx, rank_of, R)
    return dict(idx=idx, w=w, counts=counts, assign=assign, active=active, rank_of=rank_of,
                expert_offsets=expert_offsets, rank_offsets=rank_offsets, pos=pos, src=src,
                dedup=dedup)


def rows_for(meta: dict, x: np.ndarray, E: int, k: int, act_dtype: int,
             send_rows: np.ndarray | None = None, tokens: np.ndarray | None = None) -> dict:
    """Send rows, stand-in outputs and combine outputs for chosen send rows
    and tokens (all of them when None). The stand-in rows needed by the chosen
    tokens' combine are computed from their own dispatch rows."""
    T = x.shape[0]
    n = T * k
    src, pos, w = meta["src"], meta["pos"], meta["w"]
    flat_idx = meta["idx"].ravel()
    send_rows = np.arange(n) if send_rows is None else np.asarray(send_rows)
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    send = dispatch_rows(x, src, k, send_rows)
    y = expert_standin(send, flat_idx[src[send_rows]], E, act_dtype)
    # combine for the chosen tokens reads y at their k send rows; those y rows
    # are formed from their own dispatch rows and held in a compact table
    items = (tokens[:, None] * k + np.arange(k)[None, :]).ravel()
    need = pos[items]
    y_need = expert_standin(dispatch_rows(x, src, k, need), flat_idx[src[need]], E, act_dtype)
    pos_compact = np.zeros(n, dtype=np.int64)
    pos_compact[items] = np.arange(items.shape[0])
    out = combine(y_need, pos_compact, w, k, act_dtype, tokens)
    return dict(send=send, y=y, out=out, send_rows=send_rows, tokens=tokens)
