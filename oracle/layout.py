"""Dispatch layout: destination rank of each expert, segment offsets, the
stable permutation of (token, slot) pairs into send rows, and single-send
dedup counts (oracle).

Sources:
  * "METRO AllGather vs AllToAll for MoE decode", section "Work the 8-GPU
    payload example": an all-to-all cuts each rank's input into one chunk per
    destination rank; section "Distinguish METRO from backend names": a
    variable-size all-to-all is driven by per-destination counts.
  * News summary of correlated expert placement and token shuffling, section
    "Two locality techniques": a single-send dispatcher sends a token to a
    given GPU at most once.

Layout (reading taken; the pages give no buffer format): the send buffer has
exactly T*k rows (no capacity limit, nothing dropped). Rows are grouped by
destination rank; inside a rank by expert id ascending; inside an expert by
token ascending (a token never picks one expert twice, so this is also
(token, slot) order). An expert's destination rank is its assigned replica
when active, else its primary copy (it then owns zero rows).
"""
from __future__ import annotations

import numpy as np

from .replicas import candidates


def expert_ranks(E: int, R: int, rep: np.ndarray | None, assign: np.ndarray | None) -> np.ndarray:
    """rank_of[e]: destination virtual rank of expert e's rows. int32 [E]."""
    primary = np.array([c[0] for c in candidates(E, R, rep)], dtype=np.int32)
    if assign is None:
        return primary
    assign = np.asarray(assign)
    return np.where(assign >= 0, assign, primary).astype(np.int32)


def segment_offsets(counts: np.ndarray, rank_of: np.ndarray, R: int) -> tuple[np.ndarray, np.ndarray]:
    """(expert_offsets int32 [E]: first send row of expert e's segment,
    rank_offsets int32 [R+1]: first send row of each rank, last = T*k).

    Exclusive scan of the demand counts with experts taken in (rank, id)
    order: the per-destination displacements of a variable-size all-to-all."""
    counts = np.asarray(counts, dtype=np.int64)
    E = counts.shape[0]
    order = sorted(range(E), key=lambda e: (int(rank_of[e]), e))
    expert_offsets = np.zeros(E, dtype=np.int64)
    run = 0
    for e in order:
        expert_offsets[e] = run
        run += int(counts[e])
    rank_offsets = np.zeros(R + 1, dtype=np.int64)
    for r in range(R + 1):
        rank_offsets[r] = sum(int(counts[e]) for e in range(E) if rank_of[e] < r)
    return expert_offsets.astype(np.int32), rank_offsets.astype(np.int32)


def permutation(idx: np.ndarray, rank_of: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """(pos, src), both int32 [T*k]: pos[t*k + j] is the send row of token t's
    slot j, src is its inverse (send row -> flat (token, slot) index).

    Definition: list the flat pairs i = t*k + j in ascending i, stably sorted
    by their expert's place in the (rank, expert id) order; that list is src."""
    idx = np.asarray(idx)
    E = rank_of.shape[0]
    order = sorted(range(E), key=lambda e: (int(rank_of[e]), e))
    place = np.empty(E, dtype=np.int64)
    place[order] = np.arange(E)
    src = np.argsort(place[idx.ravel()], kind="stable").astype(np.int32)
    pos = np.empty_like(src)
    pos[src] = np.arange(src.shape[0], dtype=np.int32)
    return pos, src


def dedup_counts(idx: np.ndarray, rank_of: np.ndarray, R: int) -> np.ndarray:
    """dedup[r] = number of tokens with at least one selected expert whose
    rows go to rank r: the rows a single-send dispatcher sends to r. int32 [R]."""
    ranks = np.asarray(rank_of)[np.asarray(idx)]
    return np.array([np.count_nonzero((ranks == r).any(axis=1)) for r in range(R)],
                    dtype=np.int32)
