"""Router top-k, gate weights and the global expert demand vector (oracle).

Source: "METRO AllGather vs AllToAll for MoE decode", section "METRO AllGather
vs AllToAll changes the routing information": after the gather every rank runs
the same top-k over all tokens and derives one per-expert demand count.
"""
from __future__ import annotations

import numpy as np


def topk_select(logits: np.ndarray, k: int) -> np.ndarray:
    """The k experts each token selects, best first. int32 [T, k].

    The pages give top-k without a tie rule. Reading taken: expert a ranks
    above b when its logit is larger, or the logits are equal (IEEE equality,
    so -0.0 ties +0.0) and a < b; a NaN logit ranks below every number, NaNs
    among themselves by lower id. Slot 0 holds the best expert.

    Definition written out as one stable lexicographic sort per token over the
    key (is-NaN, -logit, expert id); the sort is the library step.
    """
    l = np.asarray(logits, dtype=np.float32)
    T, E = l.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    nan = np.isnan(l)
    neg = np.where(nan, 0.0, -l.astype(np.float64))
    ids = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((ids, neg, nan), axis=-1)
    return np.ascontiguousarray(order[:, :k]).astype(np.int32)


def gate_weights(logits: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Gate weight of each selected slot. float32 [T, k].

    The pages never say how gate weights are formed. Reading taken: a softmax
    over the k selected logits, w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0),
    evaluated in fp64 (l_0 is the largest selected logit, the sum runs over
    ascending slot), rounded once to fp32.
    """
    l = np.asarray(logits, dtype=np.float32).astype(np.float64)
    sel = np.take_along_axis(l, np.asarray(idx, dtype=np.int64), axis=1)
    ex = np.exp(sel - sel[:, :1])
    s = ex[:, 0].copy()
    for j in range(1, ex.shape[1]):
        s = s + ex[:, j]
    return (ex / s[:, None]).astype(np.float32)


def demand_vector(idx: np.ndarray, E: int) -> np.ndarray:
    """Global expert demand vector: counts[e] = number of (token, slot) pairs
    that selected expert e. int32 [E]; sums to T*k.

    Source: same page and section (the per-expert count every rank computes
    from the full token set)."""
    return np.bincount(np.asarray(idx).ravel(), minlength=E).astype(np.int32)
