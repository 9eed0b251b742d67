"""Single-send dispatch: one send row per (token, destination rank) instead of
one per (token, slot), and the receiver-side fan-out back to expert-grouped
rows (oracle).

Source: news summary of correlated expert placement and token shuffling,
section "Two locality techniques" (a dispatcher that sends each token to a
given GPU once; paired with correlated placement it removes dispatched rows).

Reading taken (the page gives no buffer format): the single-send buffer has
sum(dedup) rows, grouped by destination rank and inside a rank by token
ascending; the pairs (t, j) of one token whose experts live on the same rank
share that token's row for the rank. A receiver rebuilds the rank-grouped,
expert-ordered send buffer of the plain dispatch by copying each of its expert
rows from the single-send row that carries it.
"""
from __future__ import annotations

import numpy as np


def single_send_layout(idx: np.ndarray, rank_of: np.ndarray, R: int):
    """Returns (ss_rank_offsets int32 [R+1], ss_row int32 [T*k],
    ss_token int32 [n_ss]) with n_ss = ss_rank_offsets[R]."""
    idx = np.asarray(idx)
    T, k = idx.shape
    ranks = np.asarray(rank_of)[idx]                       # [T, k]
    # the distinct (rank, token) pairs in (rank, token) order are the rows
    pairs = sorted({(int(ranks[t, j]), t) for t in range(T) for j in range(k)})
    row_of = {p: q for q, p in enumerate(pairs)}
    ss_row = np.array([row_of[(int(ranks[t, j]), t)] for t in range(T) for j in range(k)],
                      dtype=np.int32)
    ss_token = np.array([t for _, t in pairs], dtype=np.int32)
    per_rank = np.bincount(np.array([r for r, _ in pairs], dtype=np.int64), minlength=R)
    ss_rank_offsets = np.concatenate([[0], np.cumsum(per_rank)]).astype(np.int32)
    return ss_rank_offsets, ss_row, ss_token


def single_send_dispatch(x: np.ndarray, ss_token: np.ndarray) -> np.ndarray:
    """send_ss[q] = x[ss_token[q]], a bit copy. [n_ss, H] uint16."""
    return x[np.asarray(ss_token)]


def single_send_expand(send_ss: np.ndarray, ss_row: np.ndarray, src: np.ndarray) -> np.ndarray:
    """Receiver fan-out: send[p] = send_ss[ss_row[src[p]]] for every row p of
    the plain (token, slot) layout. [T*k, H] uint16."""
    return send_ss[np.asarray(ss_row)[np.asarray(src)]]
