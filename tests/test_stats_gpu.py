"""GPU parity of the routing statistics against the CPU oracle, through the C
ABI, on the route and layout the GPU wrote (checked against the oracle
first): the send-counts matrix and the co-selection histogram bit-exact, and
the four summaries equal to the oracle's (exact integer sums, then the same
fp64 operations in the same order), NaN and inf included."""
import numpy as np
import pytest
import torch

import oracle
import synth
from combine_router_topk_amd import binding as B
from combine_router_topk_amd import path as P
from pathcheck import check_meta, host, run_gpu, say

pytestmark = pytest.mark.gpu


def run_stats(w, seed=0, rep="table", order="constrained", flags=0, coselect=True, logits=None):
    say(f"[case] stats {w.name} seed={seed} coselect={coselect}")
    logits = synth.make_logits(w, seed) if logits is None else logits
    x = synth.make_x(synth.scaled(w, H=8), seed)
    rep = synth.replica_table(w) if isinstance(rep, str) else rep
    ref = oracle.route_and_layout(w.T, w.E, w.k, w.R, logits, rep, order)
    b = run_gpu(synth.scaled(w, H=8), logits, x, rep, flags)
    check_meta(b, ref, w.T, w.k)
    st = P.allocate_stats(b, coselect)
    st.send_counts.fill_(-7)
    if st.coselect is not None:
        st.coselect.fill_(-7)
    P.routing_stats(b, st)
    torch.cuda.synchronize()
    S, C, stats = oracle.routing_stats(ref["idx"], ref["counts"], ref["rank_of"], w.E, w.R)
    assert np.array_equal(host(st.send_counts), S), "send_counts"
    if coselect:
        got_c = host(st.coselect)
        if not np.array_equal(got_c, C):
            bad = np.argwhere(got_c != C)[:5]
            raise AssertionError(f"coselect at {bad.tolist()}: {got_c[tuple(bad.T)]} vs {C[tuple(bad.T)]}")
    got = host(st.stats)
    assert np.array_equal(got, stats, equal_nan=True), (got.tolist(), stats.tolist())
    return got


SMALL = [
    synth.TINY,
    synth.DECODE,
    synth.scaled(synth.TRAIN_TOP2, T=3001),
    synth.scaled(synth.TRAIN_TOP6, T=2053),
    synth.scaled(synth.LARGE, T=777),
]


@pytest.mark.parametrize("seed", [0, 1])
@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_stats_small(w, seed):
    run_stats(w, seed)


@pytest.mark.parametrize("seed", [0, 1])
@pytest.mark.parametrize("w", [synth.DECODE, synth.TRAIN_TOP2, synth.TRAIN_TOP6, synth.LARGE],
                         ids=lambda w: w.name)
def test_stats_full_size(w, seed):
    got = run_stats(w, seed)
    say(f"  max/mean {got[0]:.4f} gini {got[1]:.4f} alpha {got[2]:.2f} locality {got[3]:.4f}")


EDGE = [
    ("E1_k1_R1", 50, 1, 1, 1),          # one rank: locality 1, alpha inf
    ("E8_k8_R2", 300, 8, 8, 2),         # k = E: every token holds every pair
    ("E12_k5_R3", 513, 12, 5, 3),
    ("E96_k4_R96", 800, 96, 4, 96),     # both matrices past the LDS limit
    ("E1024_k16_R1024", 300, 1024, 16, 1024),
    ("E91_k3_R7", 700, 91, 3, 7),       # C in two row slices (90 rows + 1)
    ("E1020_k8_R60", 400, 1020, 8, 60), # 128 slices of 8 rows, the last 4 rows
    ("T1", 1, 64, 2, 32),
]


@pytest.mark.parametrize("name,T,E,k,R", EDGE, ids=[e[0] for e in EDGE])
def test_stats_edge_shapes(name, T, E, k, R):
    run_stats(synth.Workload(name, T, E, k, 8, R, synth.BF16, "none", False), 5)


def test_stats_more_ranks_than_experts():
    """Expert e on rank 2e of 128 (a one-copy replica table): S lives in
    global memory while C fits in LDS."""
    E, R = 64, 128
    rep = (np.arange(E, dtype=np.int32) * 2).reshape(E, 1)
    run_stats(synth.Workload("E64_k2_R128", 999, E, 2, 8, R, synth.BF16, "none", False), 3, rep=rep)


def test_stats_slices_bounded_by_lds():
    """E = 1024 on 89 ranks (expert e on rank e mod 89): S (7921 ints) stays
    in LDS, which leaves C slices of 7 rows (146 of them, then 2 rows)."""
    E, R = 1024, 89
    rep = (np.arange(E, dtype=np.int32) % R).reshape(E, 1)
    run_stats(synth.Workload("E1024_k6_R89", 600, E, 6, 8, R, synth.BF16, "none", False), 4, rep=rep)


def test_stats_without_coselect_and_id_order():
    rng = np.random.default_rng(7)
    E, R, maxrep = 64, 8, 3
    rep = np.full((E, maxrep), -1, np.int32)
    for e in range(E):
        n = int(rng.integers(1, maxrep + 1))
        rep[e, :n] = rng.choice(R, size=n, replace=False)
    w = synth.Workload("stats_rep", 900, E, 6, 8, R, synth.F16, "zipf1.2", False)
    run_stats(w, 1, rep=rep, order="id", flags=B.MOE_FLAG_GREEDY_ID_ORDER, coselect=False)


def test_stats_uniform_locality_closed_form():
    """Logits that make token t pick expert t mod R first, with one expert per
    rank: exactly 1/8 of the pairs are local on eight ranks."""
    R = 8
    T = R * 64
    logits = np.zeros((T, R), np.float32)
    logits[np.arange(T), np.arange(T) % R] = 1.0
    w = synth.Workload("uniform8", T, R, 1, 8, R, synth.BF16, "none", False)
    got = run_stats(w, 0, logits=logits)
    assert got[3] == 0.125


def test_stats_empty_batch():
    w = synth.Workload("stats_empty", 0, 8, 2, 8, 4, synth.F16, "none", False)
    say("[case] stats empty batch")
    b = run_gpu(w, np.zeros((0, 8), np.float32), np.zeros((0, 8), np.uint16), None)
    st = P.allocate_stats(b)
    st.send_counts.fill_(-7)
    P.routing_stats(b, st)
    torch.cuda.synchronize()
    assert host(st.send_counts).sum() == 0 and host(st.coselect).sum() == 0
    assert np.isnan(host(st.stats)).all()
