"""Pins for the oracle's token-balanced (EPLB-style) split and the exhaustive
optimum: share indices against an explicit expansion, the split's structure
on random routed instances, the page's toy example, the decode-table closed
form, and a hand-worked instance where the greedy misses the optimum (no
GPU)."""
import math

import numpy as np
import pytest

import oracle
import oracle.eplb as ep
import synth
from conftest import load_golden


def test_share_index_against_expansion():
    for n in range(0, 31):
        for m in range(1, 7):
            expanded = []
            for j in range(m):
                expanded += [j] * (n // m + (1 if j < n % m else 0))
            assert len(expanded) == n
            assert [ep.replica_share_index(i, n, m) for i in range(n)] == expanded


def routed_instance(seed, T=300, E=24, k=3, R=6, maxrep=3):
    rng = np.random.default_rng(seed)
    rep = np.full((E, maxrep), -1, np.int32)
    for e in range(E):
        n = int(rng.integers(1, maxrep + 1))
        rep[e, :n] = rng.choice(R, size=n, replace=False)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    m = oracle.route_and_layout(T, E, k, R, logits, rep)
    return m, rep, E, R


@pytest.mark.parametrize("seed", range(6))
def test_split_structure(seed):
    m, rep, E, R = routed_instance(seed)
    gpu = ep.token_balanced_split(m["idx"], m["counts"], m["pos"], m["expert_offsets"], R, rep)
    flat = m["idx"].reshape(-1)
    cand = oracle.candidates(E, R, rep)
    for e in range(E):
        pairs = np.nonzero(flat == e)[0]
        order = pairs[np.argsort(m["pos"][pairs])]          # the expert's token order
        seq = [cand[e].index(int(g)) for g in gpu[order]]
        assert seq == sorted(seq)                            # contiguous shares
        n, c = int(m["counts"][e]), len(cand[e])
        assert [seq.count(j) for j in range(c)] == [n // c + (j < n % c) for j in range(c)]
    assert np.array_equal(np.bincount(gpu, minlength=R), ep.split_tokens_per_gpu(m["counts"], R, rep))
    used = {(int(flat[i]), int(gpu[i])) for i in range(flat.shape[0])}
    act = np.bincount(np.array([g for _, g in used], dtype=np.int64), minlength=R)
    assert np.array_equal(act, oracle.token_balanced_activations(m["counts"], R, rep))


def test_toy_example_split_and_optimum():
    g = load_golden("toy_16_tokens_8_gpus.json")
    rep = np.array(g["replicas"], np.int32)
    counts = np.array(g["tokens_per_expert"], np.int32)
    # expert e's two tokens go one to each of its GPUs e and e+1
    assert ep.split_tokens_per_gpu(counts, 8, rep).tolist() == [2] * 8
    assert ep.optimal_max_activated(counts, 8, rep) == 1
    _, act = oracle.greedy_assign(counts, 8, rep)
    assert act.max() == 1


def test_decode_table_all_active_closed_form():
    """Every expert active with two tokens: token balance activates both
    copies of each replicated expert, so GPU g serves its 32 own experts plus
    the 4 secondary copies it holds for GPU (g + 4) mod 8: 36. The greedy
    keeps 32, the lower bound 256 / 8, hence optimal; METRO's maximum is
    4/36 = 11.1% below token balance here. Tokens per GPU are 64 either way
    (28 experts x 2 + 4 x 1 + 4 x 1)."""
    rep = synth.replica_table(synth.DECODE)
    counts = np.full(256, 2, np.int32)
    bal = oracle.token_balanced_activations(counts, 8, rep)
    assert bal.tolist() == [36] * 8
    _, act = oracle.greedy_assign(counts, 8, rep)
    assert act.tolist() == [32] * 8 and act.max() == math.ceil(256 / 8)
    assert ep.split_tokens_per_gpu(counts, 8, rep).tolist() == [64] * 8


def test_greedy_misses_the_optimum_hand_worked():
    """Three GPUs, experts with copies {0, 2}, {1, 2}, {0, 1}, all active.
    The greedy visits them in id order (all have two copies): expert 0 ->
    GPU 0, expert 1 -> GPU 1 (ties to the lower index), expert 2 -> GPU 0
    (GPUs 0 and 1 both hold one): maximum 2. Choosing 2, 1, 0 gives one per
    GPU: the optimum is 1."""
    rep = np.array([[0, 2], [1, 2], [0, 1]], np.int32)
    counts = np.ones(3, np.int32)
    assign, act = oracle.greedy_assign(counts, 3, rep)
    assert assign.tolist() == [0, 1, 0] and act.max() == 2
    assert ep.optimal_max_activated(counts, 3, rep) == 1


@pytest.mark.parametrize("seed", range(12))
def test_optimum_bounds(seed):
    rng = np.random.default_rng(2000 + seed)
    E, R = 10, 4
    rep = np.full((E, 2), -1, np.int32)
    for e in range(E):
        n = int(rng.integers(1, 3))
        rep[e, :n] = rng.choice(R, size=n, replace=False)
    counts = ((rng.random(E) < 0.8) * rng.integers(1, 5, E)).astype(np.int32)
    n_active = int((counts > 0).sum())
    opt = ep.optimal_max_activated(counts, R, rep)
    _, act = oracle.greedy_assign(counts, R, rep)
    bal = oracle.token_balanced_activations(counts, R, rep)
    assert math.ceil(n_active / R) <= opt <= act.max(initial=0)
    assert opt <= bal.max(initial=0)   # one activated copy per expert is a valid choice
    single = rep.copy()
    single[:, 1:] = -1
    _, act1 = oracle.greedy_assign(counts, R, single)
    assert act1.max(initial=0) == ep.optimal_max_activated(counts, R, single)


def test_optimum_refuses_large_searches():
    rep = synth.replica_table(synth.DECODE)
    with pytest.raises(ValueError):
        ep.optimal_max_activated(np.ones(256, np.int32), 8, rep)


def test_greedy_gap_report():
    """The greedy against the optimum and against token balance on 300 seeded
    small instances (12 experts, 4 GPUs, one or two copies each): printed as
    the comparison the page reports; the asserts are the invariants."""
    n = n_opt = 0
    gaps, below_bal = [], []
    for seed in range(300):
        rng = np.random.default_rng(5000 + seed)
        E, R = 12, 4
        rep = np.full((E, 2), -1, np.int32)
        for e in range(E):
            m = int(rng.integers(1, 3))
            rep[e, :m] = rng.choice(R, size=m, replace=False)
        counts = ((rng.random(E) < 0.8) * rng.integers(1, 5, E)).astype(np.int32)
        if counts.sum() == 0:
            continue
        opt = ep.optimal_max_activated(counts, R, rep)
        _, act = oracle.greedy_assign(counts, R, rep)
        bal = oracle.token_balanced_activations(counts, R, rep)
        assert act.max() >= opt and bal.max() >= opt
        n += 1
        n_opt += int(act.max() == opt)
        gaps.append(act.max() / opt - 1)
        below_bal.append(1 - act.max() / bal.max())
    print(f"greedy optimal on {n_opt}/{n}; gap to optimum mean {np.mean(gaps):.3f} "
          f"max {max(gaps):.3f}; below token balance mean {np.mean(below_bal):.3f} "
          f"max {max(below_bal):.3f}")
    assert n > 250
