"""Pins for the oracle's METRO greedy replica assignment: the page's toy
example, the decode-table closed form derived by hand, a hand-worked instance,
invariants, and an exhaustive optimum on tiny instances (no GPU)."""
import math

import numpy as np
import pytest

import oracle
import synth
from conftest import load_golden


def test_toy_example_grouping_halves_activated_experts():
    g = load_golden("toy_16_tokens_8_gpus.json")
    rep = np.array(g["replicas"], np.int32)
    counts = np.array(g["tokens_per_expert"], np.int32)
    assert counts.sum() == 16
    for order in ("constrained", "id"):
        assign, act = oracle.greedy_assign(counts, g["gpus"], rep, order)
        assert act.tolist() == g["grouped_activated_per_gpu"]
        for e in range(8):
            assert assign[e] in g["replicas"][e]
    bal = oracle.token_balanced_activations(counts, g["gpus"], rep)
    assert bal.tolist() == g["token_balanced_activated_per_gpu"]
    assert bal.max() == 2 * act.max()          # the page's "halves"


@pytest.mark.parametrize("order,key", [("constrained", "active_constrained_order"),
                                       ("id", "active_id_order")])
def test_decode_table_all_active_closed_form(order, key):
    g = load_golden("decode_replica_closed_form.json")
    rep = synth.replica_table(synth.DECODE)
    counts = np.ones(256, np.int32)
    assign, act = oracle.greedy_assign(counts, 8, rep, order)
    assert act.tolist() == g[key]
    assert (assign >= 0).all()


def test_handworked_replicated_instances():
    for case in load_golden("layout_handworked.json")["cases"]:
        rep = None if case["replicas"] is None else np.array(case["replicas"], np.int32)
        assign, act = oracle.greedy_assign(np.array(case["counts"]), case["R"], rep,
                                           case.get("order", "constrained"))
        assert assign.tolist() == case["assign"], case["name"]
        assert act.tolist() == case["active"], case["name"]


def random_instance(rng, E, R, maxrep, p_active):
    rep = np.full((E, maxrep), -1, np.int32)
    for e in range(E):
        n = rng.integers(1, maxrep + 1)
        rep[e, :n] = rng.choice(R, size=n, replace=False)
    counts = (rng.random(E) < p_active) * rng.integers(1, 5, E)
    return rep, counts.astype(np.int32)


@pytest.mark.parametrize("seed", range(20))
def test_greedy_invariants(seed):
    rng = np.random.default_rng(seed)
    E, R, maxrep = int(rng.integers(1, 40)), int(rng.integers(1, 9)), int(rng.integers(1, 4))
    maxrep = min(maxrep, R)
    rep, counts = random_instance(rng, E, R, maxrep, 0.7)
    n_active = int((counts > 0).sum())
    for order in ("constrained", "id"):
        assign, act = oracle.greedy_assign(counts, R, rep, order)
        for e in range(E):
            if counts[e] > 0:
                assert assign[e] in [g for g in rep[e] if g >= 0]
            else:
                assert assign[e] == -1
        assert act.sum() == n_active
        assert act.max(initial=0) >= math.ceil(n_active / R)
        assert np.bincount(assign[assign >= 0], minlength=R).tolist() == act.tolist()


def test_no_replicas_is_per_rank_active_count():
    rng = np.random.default_rng(9)
    E, R = 64, 32
    counts = (rng.random(E) < 0.6).astype(np.int32) * 3
    assign, act = oracle.greedy_assign(counts, R, None)
    per = E // R
    for r in range(R):
        assert act[r] == sum(1 for e in range(r * per, (r + 1) * per) if counts[e] > 0)
    assert all(assign[e] == (e // per if counts[e] else -1) for e in range(E))


@pytest.mark.parametrize("seed", range(12))
def test_greedy_against_exhaustive_optimum(seed):
    rng = np.random.default_rng(1000 + seed)
    E, R = 10, 4
    rep, counts = random_instance(rng, E, R, 2, 0.8)
    _, act = oracle.greedy_assign(counts, R, rep)
    opt = oracle.optimal_max_activated(counts, R, rep)
    assert act.max() >= opt
    # single-copy experts leave no choice: greedy equals the optimum then
    single = rep.copy()
    single[:, 1:] = -1
    _, act1 = oracle.greedy_assign(counts, R, single)
    assert act1.max() == oracle.optimal_max_activated(counts, R, single)
