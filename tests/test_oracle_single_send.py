"""Pins for the oracle's single-send layout, dispatch and receiver fan-out:
hand-worked rows, brute force, special cases, and the identity that fanning
the single-send rows back out reproduces the plain dispatch (no GPU)."""
import numpy as np
import pytest

import oracle
import synth
from conftest import load_golden


def test_handworked_single_send_rows():
    for case in load_golden("layout_handworked.json")["cases"]:
        rep = None if case["replicas"] is None else np.array(case["replicas"], np.int32)
        m = oracle.route_and_layout(case["T"], case["E"], case["k"], case["R"],
                                    np.array(case["logits"], np.float32), rep,
                                    case.get("order", "constrained"))
        off, row, tok = oracle.single_send_layout(m["idx"], m["rank_of"], case["R"])
        assert off.tolist() == case["ss_rank_offsets"], case["name"]
        assert row.tolist() == case["ss_row"], case["name"]
        assert tok.tolist() == case["ss_token"], case["name"]
        assert np.diff(off).tolist() == case["dedup"]


def check(m, T, k, R, x):
    off, row, tok = oracle.single_send_layout(m["idx"], m["rank_of"], R)
    n = int(off[-1])
    assert n == int(m["dedup"].sum()) and tok.shape == (n,)
    assert np.array_equal(np.diff(off), m["dedup"])
    ranks = m["rank_of"][m["idx"]]
    seen = set()
    for t in range(T):
        for j in range(k):
            q = int(row[t * k + j])
            r = int(ranks[t, j])
            assert off[r] <= q < off[r + 1] and tok[q] == t
            seen.add((r, t))
    assert len(seen) == n                                   # one row per (token, rank)
    for r in range(R):
        assert (np.diff(tok[off[r]:off[r + 1]]) > 0).all()  # tokens ascending per rank
    send = oracle.dispatch(x, m["pos"], k)
    ss = oracle.single_send_dispatch(x, tok)
    assert np.array_equal(oracle.single_send_expand(ss, row, m["src"]), send)


@pytest.mark.parametrize("seed", range(6))
def test_random_layouts(seed):
    rng = np.random.default_rng(seed)
    E = int(rng.choice([4, 8, 16]))
    R = int(rng.choice([r for r in (1, 2, 4) if E % r == 0]))
    k = int(rng.integers(1, min(E, 5) + 1))
    T = int(rng.integers(1, 50))
    l = rng.integers(-3, 4, size=(T, E)).astype(np.float32)
    x = rng.integers(0, 65536, size=(T, 8), dtype=np.uint16)
    check(oracle.route_and_layout(T, E, k, R, l), T, k, R, x)


def test_replicated_and_workloads():
    for w in (synth.DECODE, synth.scaled(synth.TRAIN_TOP2, T=500, H=16)):
        l, x = synth.make_logits(w, 1), synth.make_x(w, 1)
        m = oracle.route_and_layout(w.T, w.E, w.k, w.R, l, synth.replica_table(w))
        check(m, w.T, w.k, w.R, x)


def test_special_cases():
    rng = np.random.default_rng(3)
    T, E, k = 40, 8, 3
    l = rng.standard_normal((T, E)).astype(np.float32)
    off, row, tok = oracle.single_send_layout(oracle.topk_select(l, k), np.zeros(E, np.int32), 1)
    assert off.tolist() == [0, T] and tok.tolist() == list(range(T))   # one rank: one row per token
    m = oracle.route_and_layout(T, E, k, E, l)                          # one expert per rank
    off, row, tok = oracle.single_send_layout(m["idx"], m["rank_of"], E)
    assert off[-1] == T * k
