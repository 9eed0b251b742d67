"""GPU parity of moe_route_assign_layout, the one-call route + greedy
assignment + layout: on every shape its outputs equal, bit for bit, those of
moe_route, moe_assign_replicas and moe_layout called in turn, and the oracle's
(idx, w, counts, assign, active, rank_of, offsets, pos, src, dedup). Decode-sized
batches take the two-launch path (top-k, then one workgroup for the rest);
larger batches, or tables too big for one workgroup's LDS, take the three
calls' kernels; both are covered."""
import numpy as np
import pytest
import torch

import oracle
import synth
from combine_router_topk_amd import binding as B
from combine_router_topk_amd import path as P
from pathcheck import bits_to_tensor, check_meta, say

pytestmark = pytest.mark.gpu

OUTPUTS = ("idx", "w", "counts", "assign", "active", "rank_of", "expert_offsets", "rank_offsets",
           "pos", "src", "dedup")


def run_both(w, seed=0, rep="table", order="constrained", logits=None):
    say(f"[case] fused plan {w.name} T={w.T} E={w.E} k={w.k} R={w.R} seed={seed} order={order}")
    logits = synth.make_logits(w, seed) if logits is None else logits
    rep = synth.replica_table(w) if isinstance(rep, str) else rep
    flags = B.MOE_FLAG_GREEDY_ID_ORDER if order == "id" else 0
    p = B.make_problem(w.T, w.E, w.k, 8, w.R, w.act_dtype, flags)
    x = bits_to_tensor(np.zeros((w.T, 8), np.uint16), w.act_dtype)
    rep_t = None if rep is None else torch.from_numpy(rep)
    a = P.allocate(p, torch.from_numpy(logits), x, rep_t)
    f = P.allocate(p, torch.from_numpy(logits), x, rep_t)
    for name in OUTPUTS:  # every output must be written by the fused call
        t = getattr(f, name)
        (t.view(torch.int32) if t.dtype == torch.float32 else t).fill_(-7)
    P.route(a)
    P.assign(a)
    P.layout(a)
    P.route_assign_layout(f)
    torch.cuda.synchronize()
    for name in OUTPUTS:
        ta, tf = getattr(a, name), getattr(f, name)
        if ta.dtype == torch.float32:
            ta, tf = ta.view(torch.int32), tf.view(torch.int32)
        assert torch.equal(ta, tf), name
    ref = oracle.route_and_layout(w.T, w.E, w.k, w.R, logits, rep, order)
    check_meta(f, ref, w.T, w.k)
    return f, ref


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_decode_two_launch_path(seed):
    f, ref = run_both(synth.DECODE, seed)
    assert int(ref["active"].max()) == 32 or seed != 0


def test_decode_id_order():
    run_both(synth.DECODE, 0, order="id")


@pytest.mark.parametrize("w", [synth.TINY, synth.scaled(synth.TRAIN_TOP2, T=4096),
                               synth.scaled(synth.TRAIN_TOP6, T=1365)], ids=lambda w: w.name)
def test_small_batches_without_table(w):
    run_both(w, 1)


# Larger batches without a replica table take three launches (top-k with
# per-block counts, a column scan, the permutation with the offset scan);
# with a table, the three calls' kernels under the one call.
@pytest.mark.parametrize("w", [synth.TRAIN_TOP2, synth.TRAIN_TOP6, synth.LARGE,
                               synth.scaled(synth.LARGE, T=20000),
                               synth.scaled(synth.TRAIN_TOP2, T=9001),
                               synth.Workload("E48_k5_R12", 12000, 48, 5, 8, 12, synth.BF16, "zipf1.2", False),
                               synth.Workload("E64_k16_R64", 20000, 64, 16, 8, 64, synth.BF16, "zipf1.2", False),
                               synth.Workload("E1024_R2_per512", 9000, 1024, 3, 8, 2, synth.BF16, "zipf1.2", False),
                               synth.Workload("E96_R96_T1M", 1 << 20, 96, 1, 8, 96, synth.BF16, "none", False)],
                         ids=lambda w: w.name)
def test_larger_batches(w):
    run_both(w, 2)


@pytest.mark.parametrize("order", ["constrained", "id"])
def test_larger_batch_with_replica_table(order):
    rng = np.random.default_rng(77)
    E, R, maxrep = 64, 16, 4
    rep = np.full((E, maxrep), -1, np.int32)
    for e in range(E):
        n = int(rng.integers(1, maxrep + 1))
        rep[e, :n] = rng.choice(R, size=n, replace=False)
    w = synth.Workload("fused_large_rep", 12000, E, 4, 8, R, synth.BF16, "cluster_pairs", False)
    run_both(w, 3, rep=rep, order=order)


@pytest.mark.parametrize("order", ["constrained", "id"])
@pytest.mark.parametrize("E,R,maxrep,T,k", [(64, 8, 3, 500, 4), (256, 128, 3, 600, 8),
                                            (100, 7, 5, 300, 6)],
                         ids=["E64_R8", "E256_R128_counters_in_LDS", "E100_R7"])
def test_random_replica_tables(order, E, R, maxrep, T, k):
    rng = np.random.default_rng(E + R)
    rep = np.full((E, maxrep), -1, np.int32)
    for e in range(E):
        n = int(rng.integers(1, min(maxrep, R) + 1))
        rep[e, :n] = rng.choice(R, size=n, replace=False)
    w = synth.Workload(f"fused_rep_E{E}_R{R}", T, E, k, 8, R, synth.BF16, "zipf1.2", False)
    run_both(w, 2, rep=rep, order=order)


EDGE = [
    ("E1_k1_R1", 50, 1, 1, 1),
    ("T1", 1, 64, 2, 32),
    ("k_equals_E", 300, 8, 8, 2),
    ("E1024_R1024_LDS_too_small", 200, 1024, 16, 1024),   # the three calls' kernels
    ("T2000_k8_past_8192_pairs", 2000, 256, 8, 32),      # the three calls' kernels
    ("T8192_k1_at_8192_pairs", 8192, 16, 1, 4),          # the largest two-launch batch
    ("T1024_k8_mask_plan_limit", 1024, 64, 8, 8),        # the largest bitmask plan
    ("T1025_k7_small_plan", 1025, 64, 7, 8),             # one token past it
    ("T300_E256_R128", 300, 256, 4, 128),                # bitmask plan, 128 ranks
]


@pytest.mark.parametrize("name,T,E,k,R", EDGE, ids=[e[0] for e in EDGE])
def test_edge_shapes(name, T, E, k, R):
    run_both(synth.Workload(name, T, E, k, 8, R, synth.F16, "none", False), 3)


def test_empty_batch():
    w = synth.Workload("empty", 0, 8, 2, 8, 4, synth.F16, "none", False)
    say("[case] fused plan empty batch")
    p = B.make_problem(0, 8, 2, 8, 4, w.act_dtype)
    f = P.allocate(p, torch.zeros(0, 8), bits_to_tensor(np.zeros((0, 8), np.uint16), w.act_dtype))
    P.route_assign_layout(f)
    torch.cuda.synchronize()
    assert f.counts.cpu().tolist() == [0] * 8 and f.assign.cpu().tolist() == [-1] * 8
    assert f.active.cpu().tolist() == [0] * 4 and f.rank_offsets.cpu().tolist() == [0] * 5
    assert f.dedup.cpu().tolist() == [0] * 4


def test_graph_of_the_fused_pass_replays_bit_for_bit():
    """The decode pass with the fused call, captured as a HIP graph: three
    replays, each on a new batch copied in place, equal the eager pass."""
    w = synth.DECODE
    rep = torch.from_numpy(synth.replica_table(w))
    p = B.make_problem(w.T, w.E, w.k, w.H, w.R, w.act_dtype)
    say("[case] fused plan graph replay")
    x0 = bits_to_tensor(synth.make_x(w, 0), w.act_dtype)
    b = P.allocate(p, torch.from_numpy(synth.make_logits(w, 0)), x0, rep)
    g = P.capture(b, P.FUSED_STEPS)
    for seed in (4, 5, 6):
        logits = torch.from_numpy(synth.make_logits(w, seed))
        x = bits_to_tensor(synth.make_x(w, seed), w.act_dtype)
        e = P.allocate(p, logits, x, rep)
        for step in P.FUSED_STEPS:
            step(e)
        b.logits.copy_(logits)
        b.x.copy_(x)
        g.replay()
        torch.cuda.synchronize()
        for name in OUTPUTS + ("send", "y", "out"):
            tb, te = getattr(b, name), getattr(e, name)
            if tb.dtype.is_floating_point:
                tb, te = tb.view(torch.int16 if tb.element_size() == 2 else torch.int32), \
                    te.view(torch.int16 if te.element_size() == 2 else torch.int32)
            assert torch.equal(tb, te), (seed, name)


def component_table(E, R, groups, maxrep, rng):
    """A replica table whose experts only list GPUs of one group, so the GPU
    graph splits into `groups` components (more or fewer than the decode
    plan's four walkers); every expert's copies are in a random order."""
    per = R // groups
    rep = np.full((E, maxrep), -1, np.int32)
    for e in range(E):
        g = e % groups
        n = int(rng.integers(1, min(maxrep, per) + 1))
        rep[e, :n] = g * per + rng.choice(per, size=n, replace=False)
    return rep


@pytest.mark.parametrize("order", ["constrained", "id"])
@pytest.mark.parametrize("groups", [1, 3, 6, 16])
def test_decode_plan_walkers_over_gpu_components(groups, order):
    """The decode plan splits the greedy walk over four waves by components of
    the GPU graph: one component (one walker), three (one walker idle), six
    and sixteen (walkers taking several) must all give the single-walker
    result, which the oracle's sequential greedy defines."""
    rng = np.random.default_rng(40 + groups)
    E, R = 96, 48
    rep = component_table(E, R, groups, 3, rng)
    w = synth.Workload(f"components{groups}", 400, E, 6, 8, R, synth.BF16, "zipf1.2", False)
    run_both(w, 7, rep=rep, order=order)


@pytest.mark.parametrize("order", ["constrained", "id"])
def test_decode_plan_without_two_copy_experts(order):
    """A table where every expert has one copy: nothing to walk in the default
    order (every walker gets no GPUs), every expert walked in the id order."""
    E, R = 64, 16
    rep = np.full((E, 2), -1, np.int32)
    rep[:, 0] = (np.arange(E) * 7) % R
    w = synth.Workload("one_copy_each", 256, E, 4, 8, R, synth.F16, "none", False)
    run_both(w, 8, rep=rep, order=order)


@pytest.mark.parametrize("order", ["constrained", "id"])
def test_decode_plan_four_column_table_with_holes(order):
    """Rows of four slots holding one to four distinct GPUs, the primary in
    slot 0 (the table's contract) and the others at random slots among 1..3
    (-1 in the rest): the decode plan's packed walk at its widest table,
    experts with four candidates included, against the separate calls and
    the oracle."""
    rng = np.random.default_rng(77)
    E, R, maxrep = 128, 32, 4
    rep = np.full((E, maxrep), -1, np.int32)
    for e in range(E):
        n = int(rng.integers(1, maxrep + 1))
        gpus = rng.choice(R, size=n, replace=False)
        rep[e, 0] = gpus[0]
        rep[e, 1 + rng.choice(maxrep - 1, size=n - 1, replace=False)] = gpus[1:]
    assert (np.sum(rep >= 0, axis=1) == 4).any()
    w = synth.Workload("four_columns_holes", 700, E, 8, 8, R, synth.BF16, "zipf1.2", False)
    run_both(w, 9, rep=rep, order=order)
