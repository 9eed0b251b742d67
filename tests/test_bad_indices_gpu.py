"""Out-of-range send positions and sources reach only the kernels' own bounds
checks: each row kernel tests every pos and src entry against the buffer it
addresses, so a corrupt entry is skipped rather than followed. Dispatch and
the single-send fan-out leave the row the slot would have written untouched; combine and dispatch
backward add nothing for it; combine backward writes no dy row and a dw of
0; the stand-in scales a row whose source is out of range as expert 0. Every
other output equals the oracle's on the same corrupted tables (the oracle
reads an appended zero row for each skipped slot, which contributes nothing
to a sum). All accesses stay inside the buffers: the corrupt values are
never used as addresses."""
import numpy as np
import pytest
import torch

import oracle
import synth
from combine_router_topk_amd import binding as B
from combine_router_topk_amd import path as P
from pathcheck import OUT_ATOL, OUT_RTOL, bits_to_tensor, host, run_gpu, say, tensor_bits

pytestmark = pytest.mark.gpu

SENTINEL = 0x7E5A
BAD_VALUES = np.array([-1, -2**31, 2**31 - 1], np.int64)


def corrupt(pos: np.ndarray, n_rows: int, rng) -> tuple[np.ndarray, np.ndarray]:
    """About 5% of the entries replaced by out-of-range values (negative,
    n_rows, n_rows + 7 and the int32 extremes); returns the table and the mask."""
    bad = rng.random(pos.shape[0]) < 0.05
    bad[0] = True  # the first token always has a corrupt slot
    vals = np.concatenate([BAD_VALUES, [n_rows, n_rows + 7]])
    out = pos.astype(np.int64).copy()
    out[bad] = vals[rng.integers(len(vals), size=int(bad.sum()))]
    return out.astype(np.int32), bad


def with_zero_row(rows: np.ndarray) -> np.ndarray:
    return np.concatenate([rows, np.zeros((1, rows.shape[1]), rows.dtype)])


SHAPES = [
    ("H264_k6", 600, 64, 6, 264, 8),     # several rows per block, combine one chunk position per step
    ("H1040_k5", 300, 32, 5, 1040, 8),   # 130 chunks: one-row blocks with the slots' rows loaded by lanes
    ("H2048_k3", 350, 16, 3, 2048, 4),   # 256 chunks: the same, at the widest such row
    ("H2056_k2", 400, 16, 2, 2056, 4),   # 257 chunks: 256-thread blocks, two chunks per lane
    ("H4104_k4", 300, 32, 4, 4104, 8),   # rows past 512 chunks
]


@pytest.mark.parametrize("name,T,E,k,H,R", SHAPES, ids=[s[0] for s in SHAPES])
def test_out_of_range_positions_are_skipped(name, T, E, k, H, R):
    rng = np.random.default_rng(11)
    w = synth.Workload(name, T, E, k, H, R, synth.BF16, "zipf1.2", False)
    logits, x = synth.make_logits(w, 3), synth.make_x(w, 3)
    say(f"[case] out-of-range positions {name}")
    ref = oracle.route_and_layout(T, E, k, R, logits)
    b = run_gpu(w, logits, x, None)
    n = T * k
    assert np.array_equal(host(b.pos), ref["pos"]) and np.array_equal(host(b.src), ref["src"])
    pos_bad, bad = corrupt(ref["pos"], n, rng)
    orphan = np.zeros(n, bool)
    orphan[ref["pos"][bad]] = True          # rows no valid slot writes
    pos_zero = np.where(bad, n, ref["pos"])  # the oracle's appended zero row
    p = B.make_problem(T, E, k, H, R, w.act_dtype)
    pos_t = torch.from_numpy(pos_bad).cuda()
    act = b.x.dtype

    # dispatch: orphaned rows untouched, the rest bit copies
    send = torch.empty_like(b.send)
    send.view(torch.int16).fill_(SENTINEL)
    B.moe_dispatch(p, b.x, pos_t, send)
    torch.cuda.synchronize()
    got = tensor_bits(send)
    assert (got[orphan] == SENTINEL).all(), "dispatch wrote a row no valid slot targets"
    keep = np.flatnonzero(~orphan)
    assert np.array_equal(got[keep], oracle.dispatch_rows(x, ref["src"], k, keep)), "dispatch rows"

    # receiver fan-out of valid single-send rows with the corrupted pos: a
    # slot whose destination is out of range writes nothing
    ss = P.allocate_single_send(b)
    P.layout_single_send(b, ss)
    P.single_send_dispatch(b, ss)
    expanded = torch.empty_like(b.send)
    expanded.view(torch.int16).fill_(SENTINEL)
    B.moe_single_send_expand(p, ss.send_ss, ss.ss_rank_offsets, ss.ss_token, ss.ss_row, pos_t,
                             expanded)
    torch.cuda.synchronize()
    got_x = tensor_bits(expanded)
    assert (got_x[orphan] == SENTINEL).all(), "fan-out wrote a row no valid slot targets"
    assert np.array_equal(got_x[keep], oracle.dispatch_rows(x, ref["src"], k, keep)), "fan-out rows"

    # combine over the GPU's y (checked elsewhere): a skipped slot adds nothing
    y_bits = tensor_bits(b.y)
    out = torch.empty_like(b.out)
    B.moe_combine(p, b.y, pos_t, b.w, out)
    torch.cuda.synchronize()
    want = oracle.combine(with_zero_row(y_bits), pos_zero, ref["w"], k, w.act_dtype)
    got_o = out.float().cpu().numpy().astype(np.float64)
    assert not (np.abs(got_o - want) > OUT_ATOL + OUT_RTOL * np.abs(want)).any(), "combine"

    # dispatch backward: a skipped slot adds nothing
    ds_bits = synth.make_grad(w, 3, n, stream=1)
    dx = torch.empty(T, H, dtype=act, device="cuda")
    B.moe_dispatch_backward(p, bits_to_tensor(ds_bits, w.act_dtype).cuda(), pos_t, dx)
    torch.cuda.synchronize()
    want = oracle.dispatch_backward(with_zero_row(ds_bits), pos_zero, k, w.act_dtype, T=T)
    got_x = dx.float().cpu().numpy().astype(np.float64)
    assert not (np.abs(got_x - want) > OUT_ATOL + OUT_RTOL * np.abs(want)).any(), "dispatch backward"

    # combine backward: no dy row for a skipped slot, its dw exactly 0
    dout = synth.make_grad(w, 3, T)
    dy = torch.empty_like(b.y)
    dy.view(torch.int16).fill_(SENTINEL)
    dw = torch.full((n,), 7.0, dtype=torch.float32, device="cuda")
    B.moe_combine_backward(p, bits_to_tensor(dout, w.act_dtype).cuda(), b.y, pos_t, b.w, dy, dw)
    torch.cuda.synchronize()
    got_dy = tensor_bits(dy)
    assert (got_dy[orphan] == SENTINEL).all(), "combine backward wrote a row no valid slot targets"
    assert np.array_equal(got_dy[keep], oracle.combine_backward_dy(dout, ref["src"], ref["w"], k,
                                                                   w.act_dtype, keep)), "dy rows"
    got_dw = host(dw).reshape(T, k).astype(np.float64)
    assert (got_dw.ravel()[bad] == 0.0).all(), "dw of a skipped slot"
    want_dw = oracle.combine_backward_dw(with_zero_row(y_bits), dout, pos_zero, k, w.act_dtype)
    mag = np.stack([(np.abs(oracle.decode16(with_zero_row(y_bits)[pos_zero[np.arange(T) * k + j]],
                                            w.act_dtype).astype(np.float64))
                     * np.abs(oracle.decode16(dout, w.act_dtype).astype(np.float64))).sum(1)
                    for j in range(k)], axis=1)
    assert not (np.abs(got_dw - want_dw) > H * 2.0 ** -24 * mag + 1e-30).any(), "dw"


def test_out_of_range_sources_read_as_expert_zero():
    rng = np.random.default_rng(12)
    T, E, k, H, R = 500, 16, 4, 520, 4
    w = synth.Workload("standin_bad_src", T, E, k, H, R, synth.F16, "none", False)
    logits, x = synth.make_logits(w, 4), synth.make_x(w, 4)
    say("[case] out-of-range stand-in sources")
    ref = oracle.route_and_layout(T, E, k, R, logits)
    b = run_gpu(w, logits, x, None)
    n = T * k
    src_bad, bad = corrupt(ref["src"], n, rng)
    y = torch.empty_like(b.y)
    B.moe_expert_standin(B.make_problem(T, E, k, H, R, w.act_dtype), b.send,
                         torch.from_numpy(src_bad).cuda(), b.idx, y)
    torch.cuda.synchronize()
    send_bits = tensor_bits(b.send)
    experts = np.where(bad, 0, ref["idx"].ravel()[np.where(bad, 0, src_bad)])
    assert np.array_equal(tensor_bits(y), oracle.expert_standin(send_bits, experts, E, w.act_dtype))


@pytest.mark.parametrize("T,E,k,R", [(900, 64, 6, 8), (5000, 256, 8, 32)], ids=["small_batch", "multi_block"])
def test_out_of_range_expert_ids_are_clamped(T, E, k, R):
    """The layout kernels clamp an expert id into [0, E): the layout of a
    corrupted idx equals the oracle's layout of the clamped ids (which may
    repeat an expert within a token). One workgroup below 8192 pairs, three
    kernels above."""
    rng = np.random.default_rng(13)
    w = synth.Workload("bad_idx", T, E, k, 8, R, synth.BF16, "zipf1.2", False)
    logits, x = synth.make_logits(w, 5), synth.make_x(w, 5)
    say(f"[case] out-of-range expert ids T={T} E={E} k={k}")
    b = run_gpu(w, logits, x, None)
    idx = host(b.idx).ravel().astype(np.int64)
    bad = rng.random(idx.shape[0]) < 0.05
    vals = np.concatenate([BAD_VALUES, [E, E + 3]])
    idx[bad] = vals[rng.integers(len(vals), size=int(bad.sum()))]
    b.idx.copy_(torch.from_numpy(idx.astype(np.int32)))
    P.layout(b)
    torch.cuda.synchronize()
    clamped = np.clip(idx, 0, E - 1).reshape(T, k)
    rank_of = oracle.expert_ranks(E, R, None, None)
    counts = oracle.demand_vector(clamped, E)
    eo, ro = oracle.segment_offsets(counts, rank_of, R)
    pos, src = oracle.permutation(clamped, rank_of)
    assert np.array_equal(host(b.rank_of), rank_of)
    assert np.array_equal(host(b.expert_offsets), eo) and np.array_equal(host(b.rank_offsets), ro)
    assert np.array_equal(host(b.pos), pos) and np.array_equal(host(b.src), src)
    assert np.array_equal(host(b.dedup), oracle.dedup_counts(clamped, rank_of, R))


@pytest.mark.parametrize("T,E,k,R", [(256, 256, 8, 8), (1500, 64, 5, 8), (12000, 64, 4, 16)],
                         ids=["bitmask_plan", "small_plan", "three_calls"])
def test_out_of_range_replica_entries_stay_in_bounds(T, E, k, R):
    """Replica entries outside [-1, R) (about 10% of them, the primary copy
    included) give an unspecified assignment, but the one-call plan keeps
    every access in bounds and its outputs well formed: assign in [-1, R)
    and only on an active expert, rank_of in [0, R), active summing to the
    experts placed, offsets consistent with the counts, pos a permutation
    of the send rows with src its inverse."""
    rng = np.random.default_rng(T + E)
    maxrep = 3
    rep = np.full((E, maxrep), -1, np.int64)
    for e in range(E):
        n = int(rng.integers(1, maxrep + 1))
        rep[e, :n] = rng.choice(R, size=n, replace=False)
    bad = rng.random(rep.shape) < 0.1
    vals = np.array([R, R + 5, -7, 2**31 - 1, -2**31], np.int64)
    rep[bad] = vals[rng.integers(len(vals), size=int(bad.sum()))]
    rep = rep.astype(np.int32)
    w = synth.Workload("bad_rep", T, E, k, 8, R, synth.BF16, "zipf1.2", False)
    say(f"[case] out-of-range replica entries T={T} E={E} k={k} R={R}")
    p = B.make_problem(T, E, k, 8, R, w.act_dtype)
    b = P.allocate(p, torch.from_numpy(synth.make_logits(w, 3)), torch.zeros(T, 8, dtype=torch.bfloat16),
                   torch.from_numpy(rep))
    P.route_assign_layout(b)
    torch.cuda.synchronize()
    counts, assign = host(b.counts), host(b.assign)
    assert counts.sum() == T * k
    assert ((assign >= -1) & (assign < R)).all()
    assert ((assign >= 0) <= (counts > 0)).all()          # only active experts are placed
    assert host(b.active).sum() == int((assign >= 0).sum())
    rank_of = host(b.rank_of)
    assert ((rank_of >= 0) & (rank_of < R)).all()
    n = T * k
    pos, src = host(b.pos).astype(np.int64), host(b.src).astype(np.int64)
    assert np.array_equal(np.sort(pos), np.arange(n)) and np.array_equal(src[pos], np.arange(n))
    ro = host(b.rank_offsets)
    assert ro[0] == 0 and ro[-1] == n
    assert np.array_equal(np.diff(ro), np.bincount(rank_of, counts, minlength=R).astype(np.int64))
