"""Token-balanced (EPLB-style) replica routing and the exact optimum of the
activated-expert objective on small instances (oracle): the two baselines the
METRO greedy is measured against.

Source: "METRO AllGather vs AllToAll for MoE decode", section "Add the
expert-weight traffic term": spreading an expert's tokens over its replicas
for token balance activates more replicas per GPU than grouping them on one
replica; the greedy is reported against the optimal maximum activated-expert
count and against EPLB's token routing.

Readings (the page names the baselines without defining them):
  * Token-balanced routing: the n tokens (slots) routed to expert e, in the
    order of e's segment of the send layout (token order), are cut into
    contiguous shares over e's m replicas in replica-table order; replica j
    takes n // m tokens, plus one more when j < n mod m. Per-replica token
    counts therefore differ by at most one, and a replica is activated when
    its share is not empty. Without a replica table every expert has one
    copy, on rank e // (E / R).
  * Optimum: the smallest possible maximum of activated experts per GPU over
    every choice of one replica per active expert, found by trying all
    choices (small instances only).
"""
from __future__ import annotations

import itertools

import numpy as np

from .replicas import candidates


def replica_share_index(i: int, n: int, m: int) -> int:
    """Replica (0..m-1) that takes the i-th of n tokens under contiguous
    shares n // m (+1 for the first n mod m replicas)."""
    q, rem = divmod(n, m)
    edge = rem * (q + 1)          # tokens held by the replicas with one more
    if i < edge:
        return i // (q + 1)
    return rem + (i - edge) // q


def token_balanced_split(idx: np.ndarray, counts: np.ndarray, pos: np.ndarray,
                         expert_offsets: np.ndarray, R: int, rep: np.ndarray | None) -> np.ndarray:
    """GPU that serves each (token, slot) pair under token-balanced routing.
    The pair's place among its expert's tokens is its row in the expert's
    send segment: pos - expert_offsets[e]. int32 [T*k]."""
    flat = np.asarray(idx).reshape(-1)
    E = np.asarray(counts).shape[0]
    cand = candidates(E, R, rep)
    out = np.empty(flat.shape[0], dtype=np.int32)
    for i, e in enumerate(flat.tolist()):
        place = int(pos[i]) - int(expert_offsets[e])
        out[i] = cand[e][replica_share_index(place, int(counts[e]), len(cand[e]))]
    return out


def split_tokens_per_gpu(counts: np.ndarray, R: int, rep: np.ndarray | None) -> np.ndarray:
    """Tokens (slots) each GPU serves under token-balanced routing. int64 [R]."""
    counts = np.asarray(counts)
    cand = candidates(counts.shape[0], R, rep)
    tok = np.zeros(R, dtype=np.int64)
    for e, c in enumerate(cand):
        q, rem = divmod(int(counts[e]), len(c))
        for j, g in enumerate(c):
            tok[g] += q + (1 if j < rem else 0)
    return tok


def optimal_max_activated(counts: np.ndarray, R: int, rep: np.ndarray | None,
                          limit: int = 1 << 20) -> int:
    """Minimum over all replica choices of the maximum activated experts per
    GPU, by trying every choice (refuses more than `limit` choices)."""
    counts = np.asarray(counts)
    cand = candidates(counts.shape[0], R, rep)
    active = [cand[e] for e in range(counts.shape[0]) if counts[e] > 0]
    n_choices = 1
    for c in active:
        n_choices *= len(c)
    if n_choices > limit:
        raise ValueError(f"{n_choices} replica choices: too many to try")
    best = None
    for choice in itertools.product(*active):
        per_gpu = np.bincount(np.array(choice, dtype=np.int64), minlength=R) if choice else [0]
        m = int(max(per_gpu))
        best = m if best is None else min(best, m)
    return best or 0
