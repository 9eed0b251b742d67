"""GPU parity of the single-send path (one send row per (token, destination
rank)) against the CPU oracle: the single-send offsets, per-slot rows and row
tokens bit-exact, every single-send row a bit copy of its token's row, rows
past the count left untouched, and the receiver fan-out equal to the plain
dispatch's send buffer, row for row."""
import numpy as np
import pytest
import torch

import oracle
import synth
from combine_router_topk_amd import binding as B
from combine_router_topk_amd import path as P
from pathcheck import bits_to_tensor, check_meta, host, say

pytestmark = pytest.mark.gpu

SENTINEL = 0x7E5A  # a 16-bit pattern no copied row can hold in every chunk


def run_single_send(w, logits, x, rep, flags=0, capacity=None):
    p = B.make_problem(w.T, w.E, w.k, w.H, w.R, w.act_dtype, flags)
    b = P.allocate(p, torch.from_numpy(logits), bits_to_tensor(x, w.act_dtype),
                   None if rep is None else torch.from_numpy(rep))
    ss = P.allocate_single_send(b)
    if capacity is not None:
        ss.send_ss = ss.send_ss[:capacity]
    ss.send_ss.view(torch.int16).fill_(SENTINEL)
    P.route(b)
    P.assign(b)
    P.layout_single_send(b, ss)
    P.dispatch(b)
    P.single_send_dispatch(b, ss)
    expanded = torch.empty_like(b.send)
    expanded.view(torch.int16).fill_(SENTINEL)
    B.moe_single_send_expand(p, ss.send_ss, ss.ss_rank_offsets, ss.ss_token, ss.ss_row, b.pos,
                             expanded)
    torch.cuda.synchronize()
    return b, ss, expanded


def rows_equal_chunked(a, b_rows_fn, n, step=1 << 15):
    for r0 in range(0, n, step):
        r1 = min(n, r0 + step)
        if not torch.equal(a[r0:r1].view(torch.int16), b_rows_fn(r0, r1).view(torch.int16)):
            return r0
    return None


def check_single_send(w, b, ss, expanded, ref, capacity=None):
    T, k = w.T, w.k
    check_meta(b, ref, T, k)
    want_off, want_row, want_tok = oracle.single_send_layout(ref["idx"], ref["rank_of"], w.R)
    n_ss = int(want_off[-1])
    assert n_ss == int(ref["dedup"].sum())
    assert np.array_equal(host(ss.ss_rank_offsets), want_off), "ss_rank_offsets"
    assert np.array_equal(host(ss.ss_row), want_row), "ss_row"
    assert np.array_equal(host(ss.ss_token)[:n_ss], want_tok), "ss_token"
    cap = ss.send_ss.shape[0]
    # every single-send row below the capacity is its token's row
    n_chk = min(n_ss, cap)
    tok = ss.ss_token[:n_chk].long()
    bad = rows_equal_chunked(ss.send_ss, lambda r0, r1: b.x.index_select(0, tok[r0:r1]), n_chk)
    assert bad is None, f"send_ss rows from {bad}"
    # rows past the count are untouched
    if cap > n_ss:
        assert bool((ss.send_ss[n_ss:].view(torch.int16) == SENTINEL).all()), "send_ss tail written"
    if capacity is None:
        # fan-out reproduces the plain dispatch exactly
        bad = rows_equal_chunked(expanded, lambda r0, r1: b.send[r0:r1], T * k)
        assert bad is None, f"expand rows from {bad}"
    else:
        # rows carried by a single-send row below the capacity are filled,
        # the others untouched
        carried = torch.from_numpy(want_row[ref["src"]] < cap).to(expanded.device)
        got, want = expanded.view(torch.int16), b.send.view(torch.int16)
        assert torch.equal(got[carried], want[carried]), "expand rows below the capacity"
        assert bool((got[~carried] == SENTINEL).all()), "expand rows past the capacity written"


SMALL = [
    synth.TINY,
    synth.DECODE,
    synth.scaled(synth.TRAIN_TOP2, T=3001, H=512),
    synth.scaled(synth.TRAIN_TOP6, T=2053, H=264),
    synth.scaled(synth.LARGE, T=777, H=7168),
]


@pytest.mark.parametrize("seed", [0, 1])
@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_single_send_small(w, seed):
    say(f"[case] single-send {w.name} seed={seed}")
    logits, x = synth.make_logits(w, seed), synth.make_x(w, seed)
    rep = synth.replica_table(w)
    ref = oracle.route_and_layout(w.T, w.E, w.k, w.R, logits, rep)
    b, ss, ex = run_single_send(w, logits, x, rep)
    check_single_send(w, b, ss, ex, ref)
    # the oracle's own fan-out agrees with its plain dispatch on sampled rows
    want_off, want_row, want_tok = oracle.single_send_layout(ref["idx"], ref["rank_of"], w.R)
    rows = np.arange(0, w.T * w.k, max(1, w.T * w.k // 64))
    got = oracle.single_send_expand(oracle.single_send_dispatch(x, want_tok), want_row, ref["src"])
    assert np.array_equal(got[rows], oracle.dispatch_rows(x, ref["src"], w.k, rows))


EDGE = [
    ("E1_k1_R1_H8", 1, 1, 1, 1, 8),          # one rank: one row per token
    ("E8_k8_R2", 300, 8, 8, 2, 16),           # every token reaches both ranks
    ("E12_k5_R3", 513, 12, 5, 3, 40),
    ("E384_k10_R12", 700, 384, 10, 12, 64),
    ("E1024_k16_R1024", 300, 1024, 16, 1024, 16),  # largest E, k and R (4-wave kernel)
    ("E64_k8_R64_T5000", 5000, 64, 8, 64, 24),     # 16-wave kernel, many rounds per block
    ("T1", 1, 64, 2, 32, 4096),
]


@pytest.mark.parametrize("name,T,E,k,R,H", EDGE, ids=[e[0] for e in EDGE])
def test_single_send_edge_shapes(name, T, E, k, R, H):
    w = synth.Workload(name, T, E, k, H, R, synth.BF16, "none", False)
    say(f"[case] single-send edge {name}")
    logits, x = synth.make_logits(w, 5), synth.make_x(w, 5)
    ref = oracle.route_and_layout(T, E, k, R, logits)
    b, ss, ex = run_single_send(w, logits, x, None)
    check_single_send(w, b, ss, ex, ref)


# Row widths (16-byte chunks per row: 129 and 256, the shapes whose
# dispatch and fan-out load the slots' rows by lanes; 257, 375, 513, 1024,
# 1537: the dispatch's long-row shapes and the fan-out's two chunks per lane).
WIDTHS = [("H1032_k3", 1032, 3), ("H2048_k6", 2048, 6), ("H2056_k3", 2056, 3),
          ("H3000_k5", 3000, 5), ("H4104_k4", 4104, 4), ("H8192_k8", 8192, 8),
          ("H12296_k7", 12296, 7)]


@pytest.mark.parametrize("name,H,k", WIDTHS, ids=[v[0] for v in WIDTHS])
def test_single_send_row_widths(name, H, k):
    w = synth.Workload(name, 300, 16, k, H, 4, synth.BF16, "zipf1.2", False)
    say(f"[case] single-send row width {name}")
    logits, x = synth.make_logits(w, 6), synth.make_x(w, 6)
    ref = oracle.route_and_layout(w.T, w.E, w.k, w.R, logits)
    b, ss, ex = run_single_send(w, logits, x, None)
    check_single_send(w, b, ss, ex, ref)


# The single-send dispatch in row slices (rows over 512 chunks, launches of
# at least 4096 slices), with ragged last slices (513 and 1537 chunks).
SLICED = [("H4104_k4_T1000", 4104, 4, 1000), ("H12296_k7_T400", 12296, 7, 400)]


@pytest.mark.parametrize("name,H,k,T", SLICED, ids=[v[0] for v in SLICED])
def test_single_send_sliced_row_widths(name, H, k, T):
    w = synth.Workload(name, T, 16, k, H, 4, synth.BF16, "zipf1.2", False)
    say(f"[case] single-send sliced row width {name}")
    logits, x = synth.make_logits(w, 7), synth.make_x(w, 7)
    ref = oracle.route_and_layout(w.T, w.E, w.k, w.R, logits)
    b, ss, ex = run_single_send(w, logits, x, None)
    check_single_send(w, b, ss, ex, ref)


@pytest.mark.parametrize("seed", [0, 1])
def test_single_send_random_replicas_id_order(seed):
    rng = np.random.default_rng(300 + seed)
    E, R, maxrep = 64, 8, 3
    rep = np.full((E, maxrep), -1, np.int32)
    for e in range(E):
        n = int(rng.integers(1, maxrep + 1))
        rep[e, :n] = rng.choice(R, size=n, replace=False)
    w = synth.Workload(f"ssrep{seed}", 900, E, 6, 64, R, synth.F16, "zipf1.2", False)
    say(f"[case] single-send random replicas seed={seed}")
    logits, x = synth.make_logits(w, seed), synth.make_x(w, seed)
    ref = oracle.route_and_layout(w.T, E, w.k, R, logits, rep, "id")
    b, ss, ex = run_single_send(w, logits, x, rep, flags=B.MOE_FLAG_GREEDY_ID_ORDER)
    check_single_send(w, b, ss, ex, ref)


def test_single_send_short_capacity_skips_rows():
    w = synth.scaled(synth.TRAIN_TOP6, T=1000, H=64)
    say("[case] single-send capacity below the row count")
    logits, x = synth.make_logits(w, 2), synth.make_x(w, 2)
    ref = oracle.route_and_layout(w.T, w.E, w.k, w.R, logits)
    n_ss = int(ref["dedup"].sum())
    b, ss, ex = run_single_send(w, logits, x, None, capacity=n_ss // 2)
    check_single_send(w, b, ss, ex, ref, capacity=n_ss // 2)


def test_single_send_empty_batch():
    w = synth.Workload("ss_empty", 0, 8, 2, 128, 4, synth.F16, "none", False)
    say("[case] single-send empty batch")
    b, ss, ex = run_single_send(w, np.zeros((0, 8), np.float32), np.zeros((0, 128), np.uint16),
                                None)
    assert host(ss.ss_rank_offsets).tolist() == [0] * 5
    assert host(b.dedup).tolist() == [0] * 4


@pytest.mark.parametrize("seed", [0, 1])
@pytest.mark.parametrize("w", [synth.DECODE, synth.TRAIN_TOP2, synth.TRAIN_TOP6, synth.LARGE],
                         ids=lambda w: w.name)
def test_single_send_full_size(w, seed):
    say(f"[case] single-send full {w.name} seed {seed}")
    logits, x = synth.make_logits(w, seed), synth.make_x(w, seed)
    rep = synth.replica_table(w)
    ref = oracle.route_and_layout(w.T, w.E, w.k, w.R, logits, rep)
    b, ss, ex = run_single_send(w, logits, x, rep)
    check_single_send(w, b, ss, ex, ref)
    say(f"  rows: plain {w.T * w.k}, single-send {int(ref['dedup'].sum())}")
