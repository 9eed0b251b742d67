"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle
on seeded synthetic inputs (every index/count/offset/row output bit-exact,
gate weights within rtol 1e-6, combine within rtol 4e-3 / atol 1e-3)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from combine_router_topk_amd import binding as B
from combine_router_topk_amd import path as P
from pathcheck import check_meta, check_rows, run_gpu, say

pytestmark = pytest.mark.gpu

# Reduced shapes: same routing structure, sizes the oracle finishes in
# seconds, several route/layout blocks and a ragged tail in tokens and in
# 16-byte row chunks.
SMALL = [
    synth.TINY,
    synth.DECODE,
    synth.scaled(synth.TRAIN_TOP2, T=3001, H=512),
    synth.scaled(synth.TRAIN_TOP6, T=2053, H=264),
    synth.scaled(synth.LARGE, T=777, H=7168),
]


def run_and_check(w, seed=0, flags=0, rep="table", order="constrained", logits=None, x=None,
                  send_rows=None, tokens=None, inplace=False):
    say(f"[case] {w.name} seed={seed} flags={flags} inplace={inplace}")
    logits = synth.make_logits(w, seed) if logits is None else logits
    x = synth.make_x(w, seed) if x is None else x
    rep = synth.replica_table(w) if isinstance(rep, str) else rep
    ref = oracle.route_and_layout(w.T, w.E, w.k, w.R, logits, rep, order)
    b = run_gpu(w, logits, x, rep, flags, inplace_standin=inplace)
    check_meta(b, ref, w.T, w.k)
    check_rows(b, ref, x, w, send_rows, tokens, out_f32=bool(flags & B.MOE_FLAG_OUT_F32),
               check_send=not inplace)
    return b, ref


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_small_workloads_all_outputs(w, seed):
    run_and_check(w, seed)


def test_decode_greedy_id_order():
    w = synth.DECODE
    b, ref = run_and_check(w, 0, flags=B.MOE_FLAG_GREEDY_ID_ORDER, order="id")
    assert ref["active"].max() >= 32


@pytest.mark.parametrize("w", [synth.TINY, synth.scaled(synth.TRAIN_TOP6, T=999, H=128),
                               synth.scaled(synth.LARGE, T=300, H=1024)], ids=lambda w: w.name)
def test_fp32_output_accumulation_bound(w):
    run_and_check(w, 1, flags=B.MOE_FLAG_OUT_F32)


def test_inplace_standin():
    run_and_check(synth.scaled(synth.TRAIN_TOP2, T=1000, H=256), 2, inplace=True)


def test_deterministic_bitwise():
    w = synth.scaled(synth.TRAIN_TOP6, T=4000, H=64)
    l, x = synth.make_logits(w, 3), synth.make_x(w, 3)
    a = run_gpu(w, l, x, None)
    b = run_gpu(w, l, x, None)
    for key in ("idx", "w", "counts", "pos", "src", "dedup", "send", "y", "out"):
        assert torch.equal(getattr(a, key).view(torch.int8) if getattr(a, key).dtype.is_floating_point
                           else getattr(a, key),
                           getattr(b, key).view(torch.int8) if getattr(b, key).dtype.is_floating_point
                           else getattr(b, key)), key


# ---- shapes at the edges of the kernels' blocking --------------------------

EDGE = [
    # route lanes per token x logits per lane in the comments
    ("E1_k1_R1_H8", 1, 1, 1, 1, 8),         # 16 x 1, one 16-byte chunk per row
    ("E5_k3_R5", 97, 5, 3, 5, 24),          # 16 x 1, padding lanes
    ("E8_k8_fullsort", 300, 8, 8, 2, 16),   # k = E
    ("E12_k5_R3", 513, 12, 5, 3, 40),       # scale 1 + e/12 not exact in binary
    ("E20_k4_R4", 257, 20, 4, 4, 8),        # 16 x 2
    ("E100_k7_R10", 611, 100, 7, 10, 72),   # 32 x 4, padded
    ("E384_k10_R12", 700, 384, 10, 12, 64), # 64 x 8, padded
    ("E1024_k16_R1024", 300, 1024, 16, 1024, 16),  # 64 x 16; largest E, k and R
    ("T1", 1, 64, 2, 32, 4096),
]


# Row widths at every launch-shape boundary of the one-row kernels (16-byte
# chunks per row): 257 and 375 (two chunks per lane, the second ragged),
# 513, 768, 1024 and 1537 (rows past 512 chunks: the 256-thread dispatch
# loops); k from 3 to 8 covers the combine's compile-time-k instances. At
# T = 300 every launch here has fewer than 4096 row slices, so none is
# sliced.
WIDTHS = [("H1024_k4", 1024, 4), ("H1032_k2", 1032, 2), ("H2048_k6", 2048, 6),
          ("H2056_k3", 2056, 3), ("H3000_k5", 3000, 5), ("H4104_k4", 4104, 4),
          ("H6144_k6", 6144, 6), ("H8192_k8", 8192, 8), ("H12296_k7", 12296, 7)]


@pytest.mark.parametrize("name,H,k", WIDTHS, ids=[v[0] for v in WIDTHS])
def test_row_widths(name, H, k):
    run_and_check(synth.Workload(name, 300, 16, k, H, 4, synth.BF16, "zipf1.2", False), 6)


# The row-slice kernels (128-chunk slices, one block each): the dispatch for
# rows over 512 chunks (launches of at least 4096 slices) or of 257-512
# chunks with k >= 5 (16384 slices), the stand-in over 512 chunks (4096),
# the combine with k >= 5 (12288), each case past every threshold it
# meets, with a ragged last slice at 375, 513 and 1537 chunks (119, 1 and
# 1 chunks), in both activation formats.
SLICED = [("H3000_k5_T5500", 3000, 5, 5500, synth.BF16), ("H4104_k6_T2500_f16", 4104, 6, 2500, synth.F16),
          ("H6144_k8_T2100", 6144, 8, 2100, synth.BF16), ("H12296_k7_T1000", 12296, 7, 1000, synth.BF16)]


@pytest.mark.parametrize("name,H,k,T,act", SLICED, ids=[v[0] for v in SLICED])
def test_sliced_row_widths(name, H, k, T, act):
    run_and_check(synth.Workload(name, T, 16, k, H, 4, act, "zipf1.2", False), 7)


@pytest.mark.parametrize("name,T,E,k,R,H", EDGE, ids=[e[0] for e in EDGE])
def test_edge_shapes(name, T, E, k, R, H):
    w = synth.Workload(name, T, E, k, H, R, synth.BF16, "none", False)
    run_and_check(w, 5)


# every route kernel shape: 16 lanes x 1 (E = 16), 32 x 4 (E = 100), one
# token per wave with 4, 8 and 16 logits per lane (E = 256, 384, 1024)
TIES = [(16, 5, 4), (100, 7, 4), (256, 8, 8), (384, 10, 12), (1024, 16, 16)]


@pytest.mark.parametrize("E,k,R", TIES, ids=[f"E{e}_k{k}" for e, k, _ in TIES])
def test_ties_signed_zeros_nan_inf(E, k, R):
    rng = np.random.default_rng(7 + E)
    T = 700
    l = rng.integers(-2, 3, size=(T, E)).astype(np.float32)
    l[rng.random((T, E)) < 0.2] = -0.0
    l[rng.random((T, E)) < 0.05] = np.nan
    l[rng.random((T, E)) < 0.02] = np.inf
    l[rng.random((T, E)) < 0.02] = -np.inf
    w = synth.Workload("ties", T, E, k, 64, R, synth.F16, "none", False)
    x = synth.make_x(w, 0)
    say(f"[case] ties T={T} E={E} k={k}")
    ref = oracle.route_and_layout(T, E, k, R, l)
    b = run_gpu(w, l, x, None)
    check_meta(b, ref, T, k)


def tie_logits(T, E, seed):
    rng = np.random.default_rng(seed)
    l = rng.integers(-2, 3, size=(T, E)).astype(np.float32)
    l[rng.random((T, E)) < 0.2] = -0.0
    l[rng.random((T, E)) < 0.05] = np.nan
    l[rng.random((T, E)) < 0.02] = np.inf
    l[rng.random((T, E)) < 0.02] = -np.inf
    return l


# ties at batch sizes with many route blocks (64-144 tokens each, the last
# one partial): E just past 128, E = 256, 384 with k = 16, and E = 1000
BIG_TIES = [(40000, 132, 3, 4), (65536, 256, 8, 8), (70000, 384, 16, 12), (36000, 1000, 1, 10)]


@pytest.mark.parametrize("T,E,k,R", BIG_TIES, ids=[f"T{t}_E{e}_k{k}" for t, e, k, _ in BIG_TIES])
def test_ties_signed_zeros_nan_inf_many_blocks(T, E, k, R):
    l = tie_logits(T, E, 11 + E)
    w = synth.Workload("ties_big", T, E, k, 64, R, synth.F16, "none", False)
    x = synth.make_x(w, 0)
    say(f"[case] ties T={T} E={E} k={k}")
    ref = oracle.route_and_layout(T, E, k, R, l)
    b = run_gpu(w, l, x, None)
    check_meta(b, ref, T, k)


def test_topk_independent_of_batch_blocking():
    """A token's ids and gate-weight bits do not depend on the batch around
    it: the first 700 tokens of a 65536-token batch (512 route blocks of
    1024 threads) equal the same 700 tokens routed alone (small blocks)."""
    T, E, k, R = 65536, 256, 8, 8
    l = tie_logits(T, E, 5)
    l[: T // 2] = np.random.default_rng(6).standard_normal((T // 2, E)).astype(np.float32)
    say("[case] top-k of a large batch against the same tokens alone")
    big = synth.Workload("big", T, E, k, 64, R, synth.F16, "none", False)
    small = synth.Workload("small", 700, E, k, 64, R, synth.F16, "none", False)
    out = []
    for wl, ll in ((big, l), (small, l[:700].copy())):
        p = B.make_problem(wl.T, wl.E, wl.k, wl.H, wl.R, wl.act_dtype)
        lt = torch.from_numpy(ll).cuda()
        idx = torch.empty(wl.T * k, dtype=torch.int32, device="cuda")
        wt = torch.empty(wl.T * k, dtype=torch.float32, device="cuda")
        counts = torch.empty(E, dtype=torch.int32, device="cuda")
        ws = torch.empty(B.moe_workspace_bytes(p), dtype=torch.uint8, device="cuda")
        B.moe_route(p, lt, idx, wt, counts, ws)
        torch.cuda.synchronize()
        out.append((idx.cpu().numpy()[: 700 * k], wt.cpu().numpy()[: 700 * k].view(np.uint32)))
    assert np.array_equal(out[0][0], out[1][0]), "idx"
    assert np.array_equal(out[0][1], out[1][1]), "w bits"


@pytest.mark.parametrize("order", ["constrained", "id"])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_random_replica_tables(order, seed):
    rng = np.random.default_rng(100 + seed)
    E, R, maxrep = 64, 8, 3
    rep = np.full((E, maxrep), -1, np.int32)
    for e in range(E):
        n = int(rng.integers(1, maxrep + 1))
        rep[e, :n] = rng.choice(R, size=n, replace=False)
    w = synth.Workload(f"rep{seed}", 500, E, 4, 64, R, synth.BF16, "zipf1.2", False)
    flags = B.MOE_FLAG_GREEDY_ID_ORDER if order == "id" else 0
    run_and_check(w, seed, flags=flags, rep=rep, order=order)


@pytest.mark.parametrize("order", ["constrained", "id"])
def test_random_replica_tables_more_than_64_gpus(order):
    """128 virtual GPUs: the greedy keeps its counters in LDS rather than in
    a register per lane."""
    rng = np.random.default_rng(321)
    E, R, maxrep = 256, 128, 3
    rep = np.full((E, maxrep), -1, np.int32)
    for e in range(E):
        n = int(rng.integers(1, maxrep + 1))
        rep[e, :n] = rng.choice(R, size=n, replace=False)
    w = synth.Workload("rep_R128", 600, E, 8, 64, R, synth.BF16, "zipf1.0_perm", False)
    flags = B.MOE_FLAG_GREEDY_ID_ORDER if order == "id" else 0
    run_and_check(w, 4, flags=flags, rep=rep, order=order)


def test_empty_batch():
    w = synth.Workload("empty", 0, 8, 2, 128, 4, synth.F16, "none", False)
    say("[case] empty batch")
    b = run_gpu(w, np.zeros((0, 8), np.float32), np.zeros((0, 128), np.uint16), None)
    assert b.counts.cpu().tolist() == [0] * 8
    assert b.assign.cpu().tolist() == [-1] * 8
    assert b.active.cpu().tolist() == [0] * 4
    assert b.rank_offsets.cpu().tolist() == [0] * 5
    assert b.expert_offsets.cpu().tolist() == [0] * 8
    assert b.dedup.cpu().tolist() == [0] * 4


def test_binding_rejects_short_buffers_and_workspace():
    w = synth.TINY
    p = B.make_problem(w.T, w.E, w.k, w.H, w.R, w.act_dtype)
    dev = torch.device("cuda")
    logits = torch.zeros(w.T, w.E, device=dev)
    idx = torch.empty(w.T * w.k, dtype=torch.int32, device=dev)
    wt = torch.empty(w.T * w.k, device=dev)
    counts = torch.empty(w.E, dtype=torch.int32, device=dev)
    small_ws = torch.empty(64, dtype=torch.uint8, device=dev)
    with pytest.raises(B.MoeError) as ei:
        B.moe_route(p, logits, idx, wt, counts, small_ws)
    assert ei.value.status == B.MOE_ERR_WORKSPACE
    with pytest.raises(ValueError):
        B.moe_route(p, logits, idx[:10], wt, counts, small_ws)


def test_two_streams_concurrently():
    """Two batches on two streams at once (the library keeps no state
    between calls): each must equal its own sequential run, bit for bit."""
    say("[case] two streams")
    ws_ = [synth.scaled(synth.TRAIN_TOP6, T=2500, H=256), synth.DECODE]
    bufs, want = [], []
    for w in ws_:
        logits, x = synth.make_logits(w, 11), synth.make_x(w, 11)
        rep = synth.replica_table(w)
        b = run_gpu(w, logits, x, rep)                  # sequential reference
        want.append({k: getattr(b, k).clone() for k in ("pos", "src", "send", "y", "out", "w")})
        for k in ("pos", "src", "send", "y", "out", "w"):
            getattr(b, k).zero_()
        bufs.append(b)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for _ in range(3):
        for b, st in zip(bufs, streams):
            with torch.cuda.stream(st):
                P.run(b)
        torch.cuda.synchronize()
        for b, wnt in zip(bufs, want):
            for k, v in wnt.items():
                got = getattr(b, k)
                assert torch.equal(got.contiguous().view(torch.uint8), v.contiguous().view(torch.uint8)), k


@pytest.mark.parametrize("reverse", [False, True], ids=["listed", "slots_reversed"])
@pytest.mark.parametrize("order", ["constrained", "id"])
def test_decode_table_all_active_full_assignment(order, reverse):
    """The assignment kernel on the all-active decode table against the
    hand-derived assignment of every expert (ties to the lower GPU index,
    whatever the order of the replica slots)."""
    from conftest import load_golden
    g = load_golden("decode_replica_closed_form.json")
    key = "two_copy_assign_constrained_order" if order == "constrained" else "two_copy_assign_id_order"
    two = {int(e): gpu for e, gpu in g[key].items()}
    expected = [two.get(e, e // 32) for e in range(256)]
    rep = synth.replica_table(synth.DECODE)
    if reverse:
        rep = np.where(rep[:, 1:2] >= 0, rep[:, ::-1], rep).astype(np.int32)
    say(f"[case] decode all-active assignment order={order} reversed={reverse}")
    w = synth.DECODE
    flags = B.MOE_FLAG_GREEDY_ID_ORDER if order == "id" else 0
    p = B.make_problem(w.T, w.E, w.k, w.H, w.R, w.act_dtype, flags)
    dev = torch.device("cuda")
    counts = torch.ones(w.E, dtype=torch.int32, device=dev)
    rep_t = torch.from_numpy(np.ascontiguousarray(rep)).to(dev)
    assign = torch.empty(w.E, dtype=torch.int32, device=dev)
    active = torch.empty(w.R, dtype=torch.int32, device=dev)
    B.moe_assign_replicas(p, counts, rep_t, rep.shape[1], assign, active)
    torch.cuda.synchronize()
    assert assign.cpu().tolist() == expected
    assert active.cpu().tolist() == g["active_constrained_order" if order == "constrained" else "active_id_order"]
