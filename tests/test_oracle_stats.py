"""Pins for the oracle's routing statistics: brute force on tiny inputs,
closed forms (equal loads, one loaded rank, the uniform locality 1/R), an
independent textbook Gini formula, a hand-worked Dirichlet fit, the moment
relation checked against numpy's Dirichlet sampler, and cross-checks with the
layout oracle (no GPU)."""
import itertools
from collections import Counter

import numpy as np
import pytest

import oracle
import oracle.stats as st
import synth


def test_send_counts_brute_force_and_layout_cross_check():
    rng = np.random.default_rng(0)
    for T, E, k, R in [(13, 8, 2, 4), (40, 12, 3, 3), (9, 6, 6, 2), (17, 16, 4, 16)]:
        logits = rng.standard_normal((T, E)).astype(np.float32)
        m = oracle.route_and_layout(T, E, k, R, logits)
        S = st.send_counts(m["idx"], m["rank_of"], R)
        want = np.zeros((R, R), np.int64)
        for t in range(T):
            s = (t * R) // T
            for j in range(k):
                want[s, m["rank_of"][m["idx"][t, j]]] += 1
        assert np.array_equal(S, want)
        # column sums are the layout's rank segment sizes
        assert np.array_equal(S.sum(0), np.diff(m["rank_offsets"]))
        # row sums are k times the tokens of each source rank
        per_src = Counter((t * R) // T for t in range(T))
        assert S.sum(1).tolist() == [k * per_src[s] for s in range(R)]


def test_coselection_brute_force():
    rng = np.random.default_rng(1)
    for T, E, k in [(20, 8, 3), (50, 16, 2), (7, 5, 5)]:
        idx = oracle.topk_select(rng.standard_normal((T, E)).astype(np.float32), k)
        C = st.coselection(idx, E)
        want = Counter()
        for t in range(T):
            for a, b in itertools.combinations(sorted(idx[t].tolist()), 2):
                want[(a, b)] += 1
        got = {(a, b): int(C[a, b]) for a in range(E) for b in range(E) if C[a, b]}
        assert got == dict(want)
        assert C.sum() == T * k * (k - 1) // 2
        assert np.tril(C).sum() == 0


def gini_sorted(x):
    """Textbook form over the ascending values x_(1..n):
    G = 2 sum_i i x_(i) / (n sum x) - (n + 1) / n."""
    x = np.sort(np.asarray(x, dtype=np.float64))
    n = x.shape[0]
    i = np.arange(1, n + 1)
    return 2.0 * (i * x).sum() / (n * x.sum()) - (n + 1.0) / n


def test_gini_closed_forms_and_textbook_formula():
    assert st.gini([5, 5, 5, 5]) == 0.0
    for R in (2, 8, 32):
        L = np.zeros(R, np.int64)
        L[3 % R] = 100
        assert st.gini(L) == pytest.approx((R - 1) / R, abs=1e-15)
    rng = np.random.default_rng(2)
    for _ in range(20):
        L = rng.integers(0, 1000, size=int(rng.integers(2, 64)))
        if L.sum() == 0:
            continue
        assert st.gini(L) == pytest.approx(gini_sorted(L), rel=1e-12, abs=1e-15)
    assert np.isnan(st.gini([0, 0, 0]))


def test_dirichlet_alpha_hand_worked_and_limits():
    # loads (3, 1): shares (3/4, 1/4), squared deviation 2 * (1/4)^2 = 1/8,
    # alpha = ((2 - 1) / (2 * 1/8) - 1) / 2 = 3/2
    assert st.dirichlet_alpha([3, 1]) == 1.5
    # loads (2, 1, 1, 0): shares (1/2, 1/4, 1/4, 0); deviations from 1/4:
    # 1/16 + 0 + 0 + 1/16 = 1/8; alpha = (3 / (4 * 1/8) - 1) / 4 = 5/4
    assert st.dirichlet_alpha([2, 1, 1, 0]) == 1.25
    assert st.dirichlet_alpha([7, 7, 7]) == float("inf")
    assert np.isnan(st.dirichlet_alpha([0, 0]))


@pytest.mark.parametrize("alpha,K", [(0.5, 8), (2.0, 8), (10.0, 32), (1.0, 64)])
def test_dirichlet_moment_relation_against_numpy_sampler(alpha, K):
    """The mean squared share deviation of symmetric Dirichlet(alpha) draws,
    inverted by the oracle's moment relation, gives alpha back."""
    rng = np.random.default_rng(int(alpha * 100) + K)
    p = rng.dirichlet(np.full(K, alpha), size=40000)
    D = ((p - 1.0 / K) ** 2).sum(axis=1).mean()
    assert st.alpha_from_sq_dev(D, K) == pytest.approx(alpha, rel=0.03)


def test_locality_closed_form_uniform_over_eight_ranks():
    """One expert per rank, token t picks expert t mod R: each source rank's
    tokens cycle through every rank equally, so exactly 1/R of the pairs are
    local (1/8 = 12.5% on eight ranks)."""
    R, m = 8, 64
    T = R * m
    idx = (np.arange(T) % R).reshape(T, 1)
    rank_of = np.arange(R)
    counts = np.bincount(idx.ravel(), minlength=R)
    S, C, stats = st.routing_stats(idx, counts, rank_of, R, R)
    assert stats[3] == 0.125
    assert stats[0] == 1.0 and stats[1] == 0.0 and stats[2] == float("inf")


def test_locality_uniform_logits_statistically():
    """i.i.d. logits over 64 experts on 8 ranks: locality ~ 1/8 (the
    standard error at T k = 80,000 pairs is about 0.0012)."""
    T, E, k, R = 40000, 64, 2, 8
    logits = np.random.default_rng(5).standard_normal((T, E)).astype(np.float32)
    m = oracle.route_and_layout(T, E, k, R, logits)
    _, _, stats = st.routing_stats(m["idx"], m["counts"], m["rank_of"], E, R)
    assert abs(stats[3] - 0.125) < 0.006


def test_single_rank_and_max_over_mean():
    idx = np.array([[0, 1], [0, 2], [0, 3], [1, 2]])
    counts = np.bincount(idx.ravel(), minlength=4)       # [3, 2, 2, 1]
    S, C, stats = st.routing_stats(idx, counts, np.zeros(4, np.int64), 4, 1)
    assert S.tolist() == [[8]]
    assert stats[0] == 3 * 4 / 8                        # max 3 over mean 2
    assert stats[1] == 0.0 and stats[2] == float("inf") and stats[3] == 1.0
    assert C[0, 1] == 1 and C[1, 2] == 1 and C[0, 3] == 1 and C.sum() == 4


def test_empty_batch_is_nan():
    idx = np.zeros((0, 2), np.int64)
    S, C, stats = st.routing_stats(idx, np.zeros(8, np.int64), np.arange(8) // 2, 8, 4)
    assert S.sum() == 0 and C.sum() == 0 and np.isnan(stats).all()


def test_top_pair_coverage():
    E = 8
    C = np.zeros((E, E), np.int64)
    C[0, 1] = 30
    C[2, 5] = 10
    C[3, 4] = 10
    # 28 pairs; 5% -> the top 2 pairs: 40 of 50
    assert st.top_pair_coverage(C, 0.05, 50) == 0.8
    assert st.top_pair_coverage(C, 1.0, 50) == 1.0


def test_clustered_workload_concentrates_pairs():
    """The train top-2 input adds +3 to expert pairs (2c, 2c+1): the 32
    cluster pairs (1.6% of 2016) hold most tokens' pairs, far above the share
    32/2016 a uniform router would give them."""
    w = synth.scaled(synth.TRAIN_TOP2, T=4000, H=8)
    m = oracle.route_and_layout(w.T, w.E, w.k, w.R, synth.make_logits(w, 0))
    C = st.coselection(m["idx"], w.E)
    cluster = sum(int(C[2 * c, 2 * c + 1]) for c in range(w.E // 2))
    assert cluster / w.T > 0.4
    assert st.top_pair_coverage(C, 32 / 2016, w.T) >= cluster / w.T


def test_hand_worked_two_ranks():
    """T = 4, E = 2 (expert e on rank e), top-1 choices (0, 0, 0, 1). Tokens
    0, 1 come from rank 0 and tokens 2, 3 from rank 1, so S = [[2, 0], [1, 1]]:
    three of four pairs are local (0.75; the diagonal entries differ). Loads
    (3, 1): Gini = 2 * 2 / (2 * 2 * 4) = 1/4; alpha = 3/2 (shares 3/4, 1/4);
    counts (3, 1) over a mean of 2: max/mean = 1.5."""
    idx = np.array([[0], [0], [0], [1]])
    S, C, stats = st.routing_stats(idx, np.array([3, 1]), np.array([0, 1]), 2, 2)
    assert S.tolist() == [[2, 0], [1, 1]]
    assert stats.tolist() == [1.5, 0.25, 1.5, 0.75]
    assert C.sum() == 0
