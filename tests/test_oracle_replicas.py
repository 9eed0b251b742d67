"""Pins for the oracle's METRO greedy replica assignment: the page's toy
example, the decode-table closed form derived by hand (per-GPU counts and the
full assignment), hand-worked instances whose replica rows list a higher GPU
before a lower one, an independent re-implementation on tiny random tables
with shuffled replica slots, invariants, and an exhaustive optimum on tiny
instances (no GPU)."""
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


@pytest.mark.parametrize("order,key", [("constrained", "two_copy_assign_constrained_order"),
                                       ("id", "two_copy_assign_id_order")])
def test_decode_table_all_active_full_assignment(order, key):
    """Every expert's GPU on the all-active decode table, derived by hand:
    single-copy experts stay on GPU e // 32, the two-copy ones as listed."""
    g = load_golden("decode_replica_closed_form.json")
    two = {int(e): gpu for e, gpu in g[key].items()}
    expected = [two.get(e, e // 32) for e in range(256)]
    assign, _ = oracle.greedy_assign(np.ones(256, np.int32), 8, synth.replica_table(synth.DECODE), order)
    assert assign.tolist() == expected


def test_handworked_ties_go_to_the_lower_gpu_not_the_first_slot():
    for case in load_golden("greedy_handworked.json")["cases"]:
        assign, act = oracle.greedy_assign(np.array(case["counts"], np.int32), case["R"],
                                           np.array(case["replicas"], np.int32), case["order"])
        assert assign.tolist() == case["assign"], case["name"]
        assert act.tolist() == case["active"], case["name"]


def greedy_by_scan(counts, R, rep, order):
    """The greedy written another way, for tiny inputs: candidate sets, the
    visiting order from buckets keyed by the number of copies, and each choice
    by scanning GPU ids upward for the first candidate at the lowest count."""
    E = len(counts)
    sets = [{int(g) for g in rep[e] if 0 <= g < R} for e in range(E)]
    live = [e for e in range(E) if counts[e] > 0 and sets[e]]
    if order == "constrained":
        buckets = {}
        for e in live:
            buckets.setdefault(len(sets[e]), []).append(e)
        live = [e for n in sorted(buckets) for e in buckets[n]]
    load, out = [0] * R, [-1] * E
    for e in live:
        lowest = min(load[g] for g in sets[e])
        g = next(g for g in range(R) if g in sets[e] and load[g] == lowest)
        out[e] = g
        load[g] += 1
    return out, load


def shuffled_slots(rng, rep):
    """The same replica sets with each row's valid entries in a random order."""
    out = rep.copy()
    for e in range(rep.shape[0]):
        n = int((rep[e] >= 0).sum())
        out[e, :n] = rng.permutation(rep[e, :n])
    return out


@pytest.mark.parametrize("seed", range(40))
def test_greedy_matches_scan_reimplementation_on_shuffled_slots(seed):
    rng = np.random.default_rng(5000 + seed)
    E, R = int(rng.integers(1, 24)), int(rng.integers(2, 7))
    maxrep = int(rng.integers(2, R + 1))
    rep, counts = random_instance(rng, E, R, maxrep, 0.8)
    rep = shuffled_slots(rng, rep)
    for order in ("constrained", "id"):
        assign, act = oracle.greedy_assign(counts, R, rep, order)
        ref_assign, ref_act = greedy_by_scan(counts, R, rep, order)
        assert assign.tolist() == ref_assign and act.tolist() == ref_act, (order, rep.tolist())


@pytest.mark.parametrize("seed", range(10))
def test_greedy_does_not_depend_on_replica_slot_order(seed):
    """Only the set of GPUs holding an expert matters to the choice (the page
    speaks of GPUs, not of a listing order); the decode table with its rows
    reversed is among the cases."""
    rng = np.random.default_rng(7000 + seed)
    if seed == 0:
        rep, counts = synth.replica_table(synth.DECODE), np.ones(256, np.int32)
        R = 8
    else:
        E, R = int(rng.integers(4, 40)), int(rng.integers(2, 9))
        rep, counts = random_instance(rng, E, R, min(3, R), 0.8)
    for order in ("constrained", "id"):
        a0, act0 = oracle.greedy_assign(counts, R, rep, order)
        for _ in range(3):
            a1, act1 = oracle.greedy_assign(counts, R, shuffled_slots(rng, rep), order)
            assert np.array_equal(a0, a1) and np.array_equal(act0, act1)


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
