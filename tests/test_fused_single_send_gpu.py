"""GPU parity of moe_route_assign_layout_single_send, the one-call route +
greedy assignment + single-send layout: on every shape its outputs equal,
bit for bit, those of moe_route, moe_assign_replicas and
moe_layout_single_send called in turn, and the oracle's (the routing, the
plain layout and the single-send offsets, rows and row tokens). Decode-sized
batches with at most 64 ranks take the two-launch path (top-k, then one
workgroup that also lays out the single-send rows); larger batches without a
replica table the three-launch path (top-k with per-rank counts and leader
masks, column scan, permutation + single-send rows); larger batches with a
table, and T = 0, the three calls' kernels."""
import numpy as np
import pytest
import torch

import oracle
import synth
from combine_router_topk_amd import binding as B
from combine_router_topk_amd import path as P
from pathcheck import bits_to_tensor, check_meta, host, say

pytestmark = pytest.mark.gpu

OUTPUTS = ("idx", "w", "counts", "assign", "active", "rank_of", "expert_offsets", "rank_offsets",
           "pos", "src", "dedup")
SS_OUTPUTS = ("ss_rank_offsets", "ss_row")


def run_both(w, seed=0, rep="table", order="constrained", logits=None):
    say(f"[case] one-call single-send plan {w.name} T={w.T} E={w.E} k={w.k} R={w.R} "
        f"seed={seed} order={order}")
    logits = synth.make_logits(w, seed) if logits is None else logits
    rep = synth.replica_table(w) if isinstance(rep, str) else rep
    flags = B.MOE_FLAG_GREEDY_ID_ORDER if order == "id" else 0
    p = B.make_problem(w.T, w.E, w.k, 8, w.R, w.act_dtype, flags)
    x = bits_to_tensor(np.zeros((w.T, 8), np.uint16), w.act_dtype)
    rep_t = None if rep is None else torch.from_numpy(rep)
    a = P.allocate(p, torch.from_numpy(logits), x, rep_t)
    f = P.allocate(p, torch.from_numpy(logits), x, rep_t)
    sa, sf = P.allocate_single_send(a), P.allocate_single_send(f)
    for name in OUTPUTS:  # every output must be written by the one call
        t = getattr(f, name)
        (t.view(torch.int32) if t.dtype == torch.float32 else t).fill_(-7)
    for name in SS_OUTPUTS + ("ss_token",):
        getattr(sf, name).fill_(-7)
        getattr(sa, name).fill_(-7)
    P.route(a)
    P.assign(a)
    P.layout_single_send(a, sa)
    P.route_assign_layout_single_send(f, sf)
    torch.cuda.synchronize()
    for name in OUTPUTS:
        ta, tf = getattr(a, name), getattr(f, name)
        if ta.dtype == torch.float32:
            ta, tf = ta.view(torch.int32), tf.view(torch.int32)
        assert torch.equal(ta, tf), name
    for name in SS_OUTPUTS:
        assert torch.equal(getattr(sa, name), getattr(sf, name)), name
    ref = oracle.route_and_layout(w.T, w.E, w.k, w.R, logits, rep, order)
    check_meta(f, ref, w.T, w.k)
    want_off, want_row, want_tok = oracle.single_send_layout(ref["idx"], ref["rank_of"], w.R)
    n_ss = int(want_off[-1])
    assert n_ss == int(ref["dedup"].sum())
    assert np.array_equal(host(sf.ss_rank_offsets), want_off), "ss_rank_offsets"
    assert np.array_equal(host(sf.ss_row), want_row), "ss_row"
    assert np.array_equal(host(sf.ss_token)[:n_ss], want_tok), "ss_token"
    assert bool((sf.ss_token[n_ss:] == -7).all()), "ss_token past the count written"
    return f, sf, ref


SMALL = [
    synth.TINY,
    synth.DECODE,                                   # replica table: the three calls' kernels
    synth.scaled(synth.TRAIN_TOP2, T=3001, H=8),
    synth.scaled(synth.TRAIN_TOP6, T=2053, H=8),
    synth.scaled(synth.LARGE, T=777, H=8),
]


@pytest.mark.parametrize("seed", [0, 1])
@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_small_workloads(w, seed):
    run_both(w, seed)


def test_decode_without_replica_table():
    run_both(synth.DECODE, 0, rep=None)


def test_decode_table_id_order():
    run_both(synth.DECODE, 0, order="id")


def test_decode_table_larger_batch():
    """1024 tokens with the decode replica table: past one workgroup's LDS,
    so the three calls' kernels."""
    run_both(synth.scaled(synth.DECODE, T=1024, H=8), 1)


@pytest.mark.parametrize("w", [synth.TRAIN_TOP2, synth.TRAIN_TOP6,
                               synth.scaled(synth.LARGE, T=40000, H=8)], ids=lambda w: w.name)
def test_full_size_batches(w):
    """T = 16384 at top-2 and top-6 (4-wave permutation blocks) and 40000
    tokens at E = 256, k = 8 (16-wave blocks, many rounds each)."""
    run_both(synth.scaled(w, H=8), 0)


EDGE = [
    ("E1_k1_R1", 1, 1, 1, 1),               # one rank: one row per token
    ("E8_k8_R2", 300, 8, 8, 2),             # every token reaches both ranks
    ("E12_k5_R3", 513, 12, 5, 3),
    ("E384_k10_R12", 700, 384, 10, 12),
    ("E1024_k16_R1024", 300, 1024, 16, 1024),  # largest E, k and R (4-wave blocks)
    ("E64_k8_R64_T5000", 5000, 64, 8, 64),
    ("E96_k4_R96_T20000", 20000, 96, 4, 96),   # rank columns past one 64-column task
    ("T1", 1, 64, 2, 32),
    ("E64_k4_R64_T1000", 1000, 64, 4, 64),    # one workgroup, 64 ranks (ballot lanes all used)
    ("E1024_k2_R32_T1000", 1000, 1024, 2, 32),  # masks too large for one workgroup: three launches
]


@pytest.mark.parametrize("name,T,E,k,R", EDGE, ids=[e[0] for e in EDGE])
def test_edge_shapes(name, T, E, k, R):
    run_both(synth.Workload(name, T, E, k, 8, R, synth.BF16, "none", False), 5, rep=None)


def test_empty_batch():
    w = synth.Workload("empty", 0, 8, 2, 8, 4, synth.F16, "none", False)
    say("[case] one-call single-send plan, empty batch")
    p = B.make_problem(0, 8, 2, 8, 4, w.act_dtype)
    b = P.allocate(p, torch.zeros((0, 8)), torch.zeros((0, 8), dtype=torch.float16))
    ss = P.allocate_single_send(b)
    P.route_assign_layout_single_send(b, ss)
    torch.cuda.synchronize()
    assert b.counts.cpu().tolist() == [0] * 8
    assert b.rank_offsets.cpu().tolist() == [0] * 5
    assert ss.ss_rank_offsets.cpu().tolist() == [0] * 5
    assert b.dedup.cpu().tolist() == [0] * 4
