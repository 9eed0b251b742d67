"""Pins for the oracle's top-k, gate weights and demand vector against brute
force, closed forms and the hand-worked example (no GPU)."""
import math
from collections import Counter

import numpy as np
import pytest

import oracle
from conftest import load_golden


def brute_topk_row(row, k):
    """Repeated selection with Python's sorted over (is-NaN, -value, id)."""
    def key(e):
        v = float(row[e])
        return (1, 0.0, e) if math.isnan(v) else (0, -v, e)
    return sorted(range(len(row)), key=key)[:k]


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("E,k", [(1, 1), (4, 2), (8, 2), (8, 8), (13, 5), (16, 16), (16, 3)])
def test_topk_brute_force_with_ties_zeros_nan(seed, E, k):
    rng = np.random.default_rng(seed * 100 + E * 7 + k)
    T = 64
    l = rng.integers(-2, 3, size=(T, E)).astype(np.float32)   # many exact ties
    l[rng.random((T, E)) < 0.15] = -0.0                          # signed zeros tie +0
    l[rng.random((T, E)) < 0.05] = np.nan
    l[rng.random((T, E)) < 0.03] = np.inf
    l[rng.random((T, E)) < 0.03] = -np.inf
    idx = oracle.topk_select(l, k)
    assert idx.dtype == np.int32 and idx.shape == (T, k)
    for t in range(T):
        assert idx[t].tolist() == brute_topk_row(l[t], k), (t, l[t])


def test_topk_full_sort_matches_stable_descending_sort():
    # k = E on finite inputs: a full stable sort by descending value
    rng = np.random.default_rng(5)
    l = rng.integers(-3, 4, size=(50, 12)).astype(np.float32)
    idx = oracle.topk_select(l, 12)
    ref = np.argsort(-l, axis=1, kind="stable")
    np.testing.assert_array_equal(idx, ref)


def test_topk_signed_zero_tie_goes_to_lower_id():
    l = np.array([[-0.0, 0.0, -1.0], [0.0, -0.0, -1.0]], np.float32)
    np.testing.assert_array_equal(oracle.topk_select(l, 1), [[0], [0]])


def test_topk_nan_below_minus_inf():
    l = np.array([[np.nan, -np.inf, np.nan, -5.0]], np.float32)
    np.testing.assert_array_equal(oracle.topk_select(l, 4), [[3, 1, 0, 2]])


def test_handworked_topk_and_counts():
    for case in load_golden("layout_handworked.json")["cases"]:
        l = np.array(case["logits"], np.float32)
        idx = oracle.topk_select(l, case["k"])
        assert idx.tolist() == case["idx"]
        assert oracle.demand_vector(idx, case["E"]).tolist() == case["counts"]


def test_weights_top2_closed_form():
    # k = 2: w0 = 1 / (1 + exp(l1 - l0)) (a logistic function of the gap)
    rng = np.random.default_rng(11)
    l = rng.standard_normal((500, 8)).astype(np.float32) * 3
    idx = oracle.topk_select(l, 2)
    w = oracle.gate_weights(l, idx)
    for t in range(500):
        l0, l1 = float(l[t, idx[t, 0]]), float(l[t, idx[t, 1]])
        w0 = 1.0 / (1.0 + math.exp(l1 - l0))
        w1 = math.exp(l1 - l0) / (1.0 + math.exp(l1 - l0))
        assert abs(w[t, 0] - w0) <= 1e-7 * w0
        assert abs(w[t, 1] - w1) <= 1e-7 * w1 + 1e-30


def test_weights_handworked_gaps():
    case = load_golden("layout_handworked.json")["cases"][0]
    l = np.array(case["logits"], np.float32)
    w = oracle.gate_weights(l, oracle.topk_select(l, 2))
    for t, gap in enumerate(case["top_gap"]):
        assert w[t, 0] == np.float32(1.0 / (1.0 + math.exp(-gap)))


@pytest.mark.parametrize("k", [1, 2, 4, 8, 16])
def test_weights_all_ties_uniform(k):
    l = np.full((3, 16), 0.75, np.float32)
    w = oracle.gate_weights(l, oracle.topk_select(l, k))
    assert (w == np.float32(1.0 / k)).all()


def test_weights_top1_is_one_and_sums_to_one():
    rng = np.random.default_rng(3)
    l = rng.standard_normal((200, 64)).astype(np.float32)
    assert (oracle.gate_weights(l, oracle.topk_select(l, 1)) == 1.0).all()
    for k in (2, 6, 8):
        w = oracle.gate_weights(l, oracle.topk_select(l, k)).astype(np.float64)
        assert np.abs(w.sum(axis=1) - 1.0).max() <= k * 2.0 ** -24
        assert (np.diff(w, axis=1) <= 0).all()   # descending logits -> descending weights


def test_weights_shift_invariant():
    # adding an integer to integer-valued logits is exact, so weights must not move
    rng = np.random.default_rng(4)
    l = rng.integers(-6, 7, size=(100, 16)).astype(np.float32)
    idx = oracle.topk_select(l, 4)
    np.testing.assert_array_equal(oracle.gate_weights(l, idx), oracle.gate_weights(l + 37.0, idx))


@pytest.mark.parametrize("seed", [0, 1])
def test_demand_vector_bruteforce_and_sum(seed):
    rng = np.random.default_rng(seed)
    T, E, k = 300, 16, 3
    l = rng.standard_normal((T, E)).astype(np.float32)
    idx = oracle.topk_select(l, k)
    c = oracle.demand_vector(idx, E)
    cnt = Counter(int(e) for e in idx.ravel())
    assert c.tolist() == [cnt.get(e, 0) for e in range(E)]
    assert c.sum() == T * k and c.max() <= T
