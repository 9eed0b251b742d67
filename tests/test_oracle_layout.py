"""Pins for the oracle's dispatch layout (segment offsets, the stable
permutation) and single-send dedup counts: hand-worked examples, brute force
with Python sorting and sets, and structural invariants (no GPU)."""
import numpy as np
import pytest

import oracle
import synth
from conftest import load_golden


def layout_of(case):
    rep = None if case["replicas"] is None else np.array(case["replicas"], np.int32)
    l = np.array(case["logits"], np.float32)
    return oracle.route_and_layout(case["T"], case["E"], case["k"], case["R"], l, rep,
                                   case.get("order", "constrained"))


def test_handworked_layouts():
    for case in load_golden("layout_handworked.json")["cases"]:
        m = layout_of(case)
        for key in ("idx", "counts", "assign", "active", "rank_of", "expert_offsets",
                    "rank_offsets", "src", "pos", "dedup"):
            assert m[key].tolist() == case[key], (case["name"], key)


def brute_src(idx, rank_of):
    T, k = idx.shape
    items = [(int(rank_of[idx[t, j]]), int(idx[t, j]), t, j) for t in range(T) for j in range(k)]
    return [it[2] * k + it[3] for it in sorted(items)]


def brute_dedup(idx, rank_of, R):
    d = [0] * R
    for t in range(idx.shape[0]):
        for r in {int(rank_of[e]) for e in idx[t]}:
            d[r] += 1
    return d


def check_structure(m, T, k, R):
    n = T * k
    pos, src, idx = m["pos"], m["src"], m["idx"]
    counts, rank_of = m["counts"], m["rank_of"]
    assert np.array_equal(np.sort(pos), np.arange(n))           # bijection
    assert np.array_equal(src[pos], np.arange(n))               # inverse
    flat = idx.ravel()
    E = counts.shape[0]
    for e in range(E):
        a, c = int(m["expert_offsets"][e]), int(counts[e])
        seg = src[a:a + c]
        assert (flat[seg] == e).all()                           # segment holds only e
        assert (np.diff(seg) > 0).all()                         # (token, slot) order
        r = rank_of[e]
        assert m["rank_offsets"][r] <= a and a + c <= m["rank_offsets"][r + 1]
    ro = m["rank_offsets"]
    assert ro[0] == 0 and ro[-1] == n and (np.diff(ro) >= 0).all()
    for r in range(R):
        assert ro[r + 1] - ro[r] == counts[rank_of == r].sum()
    d = m["dedup"].sum()
    assert T <= d <= n or T == 0


@pytest.mark.parametrize("seed", range(10))
def test_layout_bruteforce_random(seed):
    rng = np.random.default_rng(seed)
    E = int(rng.choice([2, 4, 8, 12, 16]))
    R = int(rng.choice([r for r in (1, 2, 4) if E % r == 0]))
    k = int(rng.integers(1, min(E, 5) + 1))
    T = int(rng.integers(1, 40))
    l = rng.integers(-3, 4, size=(T, E)).astype(np.float32)
    m = oracle.route_and_layout(T, E, k, R, l)
    assert m["src"].tolist() == brute_src(m["idx"], m["rank_of"])
    assert m["dedup"].tolist() == brute_dedup(m["idx"], m["rank_of"], R)
    check_structure(m, T, k, R)


@pytest.mark.parametrize("seed", range(6))
def test_layout_bruteforce_replicated(seed):
    rng = np.random.default_rng(50 + seed)
    E, R, T, k = 12, 4, 30, 3
    rep = np.full((E, 2), -1, np.int32)
    for e in range(E):
        rep[e, 0] = e % R
        if rng.random() < 0.5:
            rep[e, 1] = (e + 1 + rng.integers(0, R - 1)) % R
    l = rng.standard_normal((T, E)).astype(np.float32)
    for order in ("constrained", "id"):
        m = oracle.route_and_layout(T, E, k, R, l, rep, order)
        assert m["src"].tolist() == brute_src(m["idx"], m["rank_of"])
        assert m["dedup"].tolist() == brute_dedup(m["idx"], m["rank_of"], R)
        check_structure(m, T, k, R)
        # inactive experts sit on their primary copy with zero rows
        for e in range(E):
            if m["counts"][e] == 0:
                assert m["assign"][e] == -1 and m["rank_of"][e] == rep[e, 0]


def test_dedup_special_cases():
    rng = np.random.default_rng(7)
    T, E = 200, 8
    l = rng.standard_normal((T, E)).astype(np.float32)
    # one rank: every token is sent once
    m = oracle.route_and_layout(T, E, 3, 1, l)
    assert m["dedup"].tolist() == [T]
    # one expert per rank: nothing to merge, T*k rows
    m = oracle.route_and_layout(T, E, 3, E, l)
    assert m["dedup"].sum() == T * 3


def test_workload_layouts_structure():
    for w in (synth.TINY, synth.DECODE, synth.TRAIN_TOP2):
        l = synth.make_logits(w, 0)
        m = oracle.route_and_layout(w.T, w.E, w.k, w.R, l, synth.replica_table(w))
        check_structure(m, w.T, w.k, w.R)
        assert m["counts"].sum() == w.T * w.k


def test_empty_batch():
    l = np.zeros((0, 8), np.float32)
    m = oracle.route_and_layout(0, 8, 2, 4, l)
    assert m["idx"].shape == (0, 2) and m["pos"].shape == (0,)
    assert m["counts"].tolist() == [0] * 8 and m["active"].tolist() == [0] * 4
    assert m["rank_offsets"].tolist() == [0] * 5 and m["dedup"].tolist() == [0] * 4
    assert (m["assign"] == -1).all()


def test_inactive_experts_sit_on_their_first_listed_copy():
    """Worked by hand: an expert without rows keeps its primary copy (the
    first entry of its replica row, here a higher GPU than its second copy),
    not its lowest or last-listed one; with no rows it moves no offset.
    E = 4 on 3 GPUs, rows [[2, 0], [1, -], [0, 2], [1, 2]], counts [0, 5, 0, 3]:
    expert 1 (one copy) goes to GPU 1, expert 3 to GPU 2 (0 activated against
    1); experts 0 and 2 are inactive and sit on GPUs 2 and 0. Send order
    (rank, id): expert 2 (0 rows), expert 1 (5), expert 0 (0), expert 3 (3)."""
    rep = np.array([[2, 0], [1, -1], [0, 2], [1, 2]], np.int32)
    counts = np.array([0, 5, 0, 3], np.int32)
    assign, act = oracle.greedy_assign(counts, 3, rep)
    assert assign.tolist() == [-1, 1, -1, 2] and act.tolist() == [0, 1, 1]
    rank_of = oracle.expert_ranks(4, 3, rep, assign)
    assert rank_of.tolist() == [2, 1, 0, 2]
    eo, ro = oracle.segment_offsets(counts, rank_of, 3)
    assert eo.tolist() == [5, 0, 0, 5] and ro.tolist() == [0, 0, 5, 8]
