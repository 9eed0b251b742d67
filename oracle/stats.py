"""Routing statistics of one batch (oracle): the send-counts matrix, the
co-selection pair histogram, and four scalar summaries.

Sources:
  * "Diagnosing Overhead in Dispatch Operations: Cross-architecture
    Observatory", section "Methodology": three scalar summaries of the
    send-counts matrix S (a per-expert max/mean ratio for routing skew, a Gini
    coefficient for per-rank load imbalance, and a fitted symmetric Dirichlet
    alpha for near-uniform regimes).
  * News summary of correlated expert placement and token shuffling, section
    "Correlations in router choices" (expert pairs selected together by the
    same token) and section "Two locality techniques" (the share of
    token-to-expert assignments served on the token's own GPU, 12.5% before
    shuffling on eight GPUs).

Readings (the pages give names, not formulas):
  * Token t comes from virtual rank floor(t * R / T) (contiguous, balanced
    shards of the batch); S[s, d] counts the (token, slot) pairs from source
    rank s whose expert sits on rank d (the rows an all-to-all sends from s to
    d). The per-rank load is the column sum L[d] = sum_s S[s, d].
  * max/mean = max_e counts[e] / (T k / E).
  * Gini over the R per-rank loads: sum_i sum_j |L_i - L_j| / (2 R sum_i L_i).
  * Dirichlet alpha: the per-rank shares p = L / sum(L) taken as one draw of
    a symmetric Dirichlet over K = R categories and fitted by moments. For
    that distribution E[sum_i (p_i - 1/K)^2] = (K - 1) / (K (K alpha + 1)), so
    alpha = ((K - 1) / (K D) - 1) / K with D the observed sum of squared
    deviations; +inf when D = 0 (all loads equal).
  * locality = trace(S) / sum(S): the share of pairs whose expert sits on
    the token's own rank.
  * The co-selection histogram C[a, b] (a < b) counts tokens that selected
    both a and b; entries with a >= b are 0.
  * With T = 0 every ratio is 0/0 and is returned as NaN.
"""
from __future__ import annotations

import numpy as np


def source_ranks(T: int, R: int) -> np.ndarray:
    """Virtual source rank of each token: floor(t R / T)."""
    return (np.arange(T, dtype=np.int64) * R // max(T, 1)).astype(np.int64)


def send_counts(idx: np.ndarray, rank_of: np.ndarray, R: int) -> np.ndarray:
    """S [R, R] int64: pairs by (source rank of the token, rank of the expert)."""
    idx = np.asarray(idx)
    T, k = idx.shape
    S = np.zeros((R, R), dtype=np.int64)
    src = np.repeat(source_ranks(T, R), k)
    dst = np.asarray(rank_of)[idx.reshape(-1)]
    np.add.at(S, (src, dst), 1)
    return S


def coselection(idx: np.ndarray, E: int) -> np.ndarray:
    """C [E, E] int64: C[a, b] for a < b is the number of tokens whose k
    selected experts include both a and b."""
    idx = np.asarray(idx)
    T, k = idx.shape
    C = np.zeros((E, E), dtype=np.int64)
    for i in range(k):
        for j in range(i + 1, k):
            a, b = idx[:, i], idx[:, j]
            np.add.at(C, (np.minimum(a, b), np.maximum(a, b)), 1)
    return C


def gini(loads: np.ndarray) -> float:
    """Gini coefficient: mean absolute difference over twice the mean."""
    L = np.asarray(loads, dtype=np.int64)
    n, tot = L.shape[0], int(L.sum())
    if tot == 0:
        return float("nan")
    num = int(np.abs(L[:, None] - L[None, :]).sum())
    return num / (2.0 * n * tot)


def alpha_from_sq_dev(D: float, K: int) -> float:
    """Symmetric Dirichlet alpha whose expected sum of squared share
    deviations from 1/K equals D."""
    if D == 0:
        return float("inf")
    return ((K - 1) / (K * D) - 1.0) / K


def dirichlet_alpha(loads: np.ndarray) -> float:
    """Moment fit of a symmetric Dirichlet to the shares of `loads`. The
    squared deviation is formed exactly in integers:
    sum_i (L_i / N - 1/K)^2 = (K sum_i L_i^2 - N^2) / (K N^2)."""
    L = np.asarray(loads, dtype=np.int64)
    K, N = L.shape[0], int(L.sum())
    if N == 0:
        return float("nan")
    num = K * int((L * L).sum()) - N * N
    if num == 0:
        return float("inf")
    D = num / (K * float(N) * N)
    return alpha_from_sq_dev(D, K)


def routing_stats(idx: np.ndarray, counts: np.ndarray, rank_of: np.ndarray, E: int, R: int):
    """(S, C, stats) with stats = [max/mean, gini, alpha, locality] (float64)."""
    idx = np.asarray(idx)
    T, k = idx.shape
    S = send_counts(idx, rank_of, R)
    C = coselection(idx, E)
    N = T * k
    loads = S.sum(axis=0)
    nan = float("nan")
    stats = np.array([
        int(np.max(counts)) * E / float(N) if N else nan,
        gini(loads),
        dirichlet_alpha(loads),
        int(np.trace(S)) / float(N) if N else nan,
    ], dtype=np.float64)
    return S, C, stats


def top_pair_coverage(C: np.ndarray, frac_pairs: float, T: int) -> float:
    """Share of the tokens' selected pairs held by the most frequent
    ceil(frac_pairs * E (E - 1) / 2) expert pairs (at top-2 each token has one
    pair, so this is the share of tokens)."""
    E = C.shape[0]
    n_pairs = E * (E - 1) // 2
    iu = np.triu_indices(E, 1)
    vals = np.sort(C[iu])[::-1]
    m = int(np.ceil(frac_pairs * n_pairs))
    tot = int(vals.sum())
    return float(vals[:m].sum()) / tot if tot else float("nan")
