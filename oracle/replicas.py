"""METRO greedy replica assignment (oracle).

Source: "METRO AllGather vs AllToAll for MoE decode":
  * section "METRO AllGather vs AllToAll changes the routing information":
    every active expert (demand > 0) is served by exactly one of its replicas,
    the one on the GPU that so far has the fewest activated experts; the aim
    is a small maximum number of activated experts per GPU;
  * section "Add the expert-weight traffic term": the assignment is greedy,
    not the expensive optimum, and the toy example (16 tokens on 8 GPUs)
    shows grouping an expert's tokens on one replica halving the activated
    experts per GPU compared with spreading them for token balance.

Readings taken where the pages are open:
  * Processing order. Default: most-constrained first, i.e. active experts in
    ascending (number of replicas, expert id). Experts with a single replica
    have no choice and are activated wherever they live, so they are counted
    before any choice is made. The literal ascending-id order is kept as an
    option ("id"); on the replicated decode table with every expert active it
    gives GPUs of 29 and 35 activated experts, worse than 32 without replicas,
    which contradicts the stated aim.
  * "Fewest" ties go to the lowest virtual-GPU index (not the replica slot).
  * Inactive experts get no replica (-1) and do not count as activated.
"""
from __future__ import annotations

import numpy as np


def candidates(E: int, R: int, rep: np.ndarray | None) -> list[list[int]]:
    """Virtual GPUs that hold a copy of each expert. Without a replica table
    the experts are split contiguously: expert e lives on rank e // (E / R)."""
    if rep is None:
        if E % R:
            raise ValueError("contiguous partition needs R | E")
        per = E // R
        return [[e // per] for e in range(E)]
    rep = np.asarray(rep)
    return [[int(g) for g in rep[e] if g >= 0] for e in range(E)]


def greedy_assign(counts: np.ndarray, R: int, rep: np.ndarray | None,
                  order: str = "constrained") -> tuple[np.ndarray, np.ndarray]:
    """Returns (assign int32 [E] with -1 for inactive experts,
    active int32 [R] = activated experts per virtual GPU)."""
    counts = np.asarray(counts)
    E = counts.shape[0]
    cand = candidates(E, R, rep)
    act_experts = [e for e in range(E) if counts[e] > 0]
    if order == "constrained":
        act_experts.sort(key=lambda e: (len(cand[e]), e))
    elif order != "id":
        raise ValueError("order must be 'constrained' or 'id'")
    active = [0] * R
    assign = [-1] * E
    for e in act_experts:
        g = min(cand[e], key=lambda g: (active[g], g))
        assign[e] = g
        active[g] += 1
    return np.array(assign, dtype=np.int32), np.array(active, dtype=np.int32)


def token_balanced_activations(tokens_per_expert: np.ndarray, R: int,
                               rep: np.ndarray | None) -> np.ndarray:
    """Activated experts per GPU when each expert's tokens are spread over all
    of its replicas as evenly as possible (the token-balance routing that the
    toy example contrasts with grouping): replica i of expert e gets
    ceil/floor shares, and every replica with at least one token is active."""
    tokens_per_expert = np.asarray(tokens_per_expert)
    E = tokens_per_expert.shape[0]
    cand = candidates(E, R, rep)
    active = np.zeros(R, dtype=np.int32)
    for e in range(E):
        n, c = int(tokens_per_expert[e]), cand[e]
        for i, g in enumerate(c):
            share = n // len(c) + (1 if i < n % len(c) else 0)
            if share > 0:
                active[g] += 1
    return active
