"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times: every index output compared whole with the oracle; every
stand-in row bit for bit and every combine output element within tolerance,
token chunk by token chunk (the oracle run on a thread pool); and the dispatch
identity send[r] == x[src[r] / k] checked on every row on the GPU (with src
equal to the oracle's, that is every send row equal to the oracle's)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from pathcheck import check_meta, check_rows_all, run_gpu, say

pytestmark = pytest.mark.gpu


def sample(rng, n, m):
    s = rng.choice(n, size=min(m, n), replace=False)
    return np.unique(np.concatenate([s, [0, n - 1]])).astype(np.int64)


def dispatch_identity_all_rows(b, k):
    rows = b.send.shape[0]
    step = 1 << 16
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        tok = (b.src[r0:r1].long() // k)
        assert torch.equal(b.send[r0:r1].view(torch.int16), b.x.index_select(0, tok).view(torch.int16)), r0


# every workload at seeds 0-2
FULL_CASES = [(w, s) for w in (synth.DECODE, synth.TRAIN_TOP2, synth.TRAIN_TOP6, synth.LARGE) for s in (0, 1, 2)]


@pytest.mark.parametrize("w,seed", FULL_CASES, ids=lambda v: v.name if hasattr(v, "name") else f"seed{v}")
def test_full_size(w, seed):
    say(f"[case] full {w.name} seed {seed}")
    logits = synth.make_logits(w, seed)
    x = synth.make_x(w, seed)
    rep = synth.replica_table(w)
    ref = oracle.route_and_layout(w.T, w.E, w.k, w.R, logits, rep)
    b = run_gpu(w, logits, x, rep)
    check_meta(b, ref, w.T, w.k)
    dispatch_identity_all_rows(b, w.k)
    check_rows_all(b, ref, x, w)
    assert int(b.counts.sum()) == w.T * w.k


def test_max_rows():
    """T*k at the row limit, 2^24 - 16 rows (T = 2^20 - 1, k = 16), with
    64-chunk rows: the stand-in launches one 256-thread block per send row,
    4,294,963,200 work-items, just under the 2^32 a launch holds. At this
    size the oracle computes the sampled tokens one by one (top-k, gate
    weights, stand-in rows, combine) from the logits and activations; the
    index outputs are checked whole against properties that fix them: counts
    and dedup by their definitions, pos a permutation with src its inverse
    whose (rank, expert, token) keys strictly increase, offsets the
    exclusive sums of the counts in that order; and the dispatch identity
    on every row."""
    from combine_router_topk_amd import binding as B
    T, k, E, R, H = (1 << 20) - 1, 16, 64, 32, 512
    assert T * k <= B.MOE_MAX_ROWS
    w = synth.Workload("max_rows_T1048575_E64_k16_H512", T, E, k, H, R, synth.BF16, "zipf1.2", False)
    say(f"[case] {w.name}: {T * k} rows")
    logits = synth.make_logits(w, 0)
    x = synth.make_x(w, 0)
    b = run_gpu(w, logits, x, None)
    idx = b.idx.cpu().numpy().reshape(T, k)
    rng = np.random.default_rng(99)
    toks = sample(rng, T, 512)
    ref_idx = oracle.topk_select(logits[toks], k)
    assert np.array_equal(idx[toks], ref_idx), "idx on sampled tokens"
    ref_w = oracle.gate_weights(logits[toks], ref_idx).astype(np.float64)
    got_w = b.w.cpu().numpy().reshape(T, k)[toks].astype(np.float64)
    assert (np.abs(got_w - ref_w) <= 1e-6 * np.abs(ref_w)).all(), "w on sampled tokens"
    counts = b.counts.cpu().numpy()
    assert np.array_equal(counts, np.bincount(idx.ravel(), minlength=E)), "counts"
    rank_of = b.rank_of.cpu().numpy()
    assert np.array_equal(rank_of, np.arange(E) // (E // R)), "rank_of"
    pos, src = b.pos.cpu().numpy().astype(np.int64), b.src.cpu().numpy().astype(np.int64)
    n = T * k
    assert np.array_equal(np.sort(pos), np.arange(n)), "pos is a permutation"
    assert np.array_equal(src[pos], np.arange(n)), "src inverts pos"
    e_r = idx.ravel()[src]
    key = (rank_of[e_r].astype(np.int64) * E + e_r) * T + src // k
    assert (np.diff(key) > 0).all(), "rows ordered by (rank, expert, token)"
    order = np.lexsort((np.arange(E), rank_of))
    starts = np.zeros(E, np.int64)
    starts[order] = np.concatenate([[0], np.cumsum(counts[order])[:-1]])
    assert np.array_equal(b.expert_offsets.cpu().numpy(), starts), "expert_offsets"
    roff = b.rank_offsets.cpu().numpy()
    assert np.array_equal(roff, np.concatenate([[0], np.cumsum(np.bincount(rank_of, counts, R))]).astype(roff.dtype)), "rank_offsets"
    ranks = rank_of[idx]
    dedup = np.bincount(np.concatenate([np.unique(ranks[t0:t0 + 4096] + R * np.arange(t0, min(T, t0 + 4096))[:, None])
                                        for t0 in range(0, T, 4096)]) % R, minlength=R)
    assert np.array_equal(b.dedup.cpu().numpy(), dedup), "dedup"
    dispatch_identity_all_rows(b, k)
    # stand-in rows and combine outputs of the sampled tokens, from scratch
    xs = x[toks]
    yref = oracle.expert_standin(np.repeat(xs, k, axis=0), ref_idx.ravel(), E, w.act_dtype)
    rows_t = torch.from_numpy(pos.reshape(T, k)[toks].ravel()).to(b.y.device)
    got_y = b.y.index_select(0, rows_t).cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got_y, yref), "stand-in rows of sampled tokens"
    out_ref = oracle.combine(yref, np.arange(toks.shape[0] * k), ref_w.astype(np.float32), k, w.act_dtype)
    got = b.out.index_select(0, torch.from_numpy(toks).to(b.out.device)).float().cpu().numpy().astype(np.float64)
    assert (np.abs(got - out_ref) <= 1e-3 + 4e-3 * np.abs(out_ref)).all(), "combine of sampled tokens"


def test_wide_rows_over_several_dispatch_launches():
    """Rows of 2048 chunks (H = 16384) go out in 16 slices of 128 chunks, one
    block each, and one launch takes at most 2^22 such blocks: T = 262200
    tokens make 4,195,200 of them, so the dispatch and the single-send
    dispatch each run as two launches (262144 tokens, then 56). The index
    outputs are compared whole with the oracle; every send row, and every
    single-send row, is checked against its token's row on the GPU. The
    activations (8.6 GB) are drawn on the GPU (seeded): only these
    identities use them."""
    from combine_router_topk_amd import binding as B
    from combine_router_topk_amd import path as P
    T, E, k, H, R = 262200, 8, 1, 16384, 4
    w = synth.Workload(f"wide_T{T}_E{E}_k{k}_H{H}", T, E, k, H, R, synth.BF16, "zipf1.2", False)
    say(f"[case] {w.name}: sliced dispatch over two launches")
    logits = synth.make_logits(w, 0)
    g = torch.Generator(device="cuda").manual_seed(5)
    x = torch.empty(T, H, dtype=torch.bfloat16, device="cuda")
    for t0 in range(0, T, 1 << 15):  # drawn in pieces to bound the fp32 temporaries
        t1 = min(T, t0 + (1 << 15))
        x[t0:t1] = torch.randn(t1 - t0, H, generator=g, device="cuda").to(torch.bfloat16)
    p = B.make_problem(T, E, k, H, R, B.MOE_BF16)
    b = P.allocate(p, torch.from_numpy(logits), x)
    del x
    b.y = b.out = None  # not used here
    torch.cuda.empty_cache()
    b.send.fill_(7.0)
    P.route_assign_layout(b)
    P.dispatch(b)
    ss = P.allocate_single_send(b)
    P.layout_single_send(b, ss)
    ss.send_ss.fill_(7.0)
    P.single_send_dispatch(b, ss)
    torch.cuda.synchronize()
    ref = oracle.route_and_layout(T, E, k, R, logits, None)
    check_meta(b, ref, T, k)
    dispatch_identity_all_rows(b, k)
    n_ss = int(ss.ss_rank_offsets[R])
    assert n_ss == int(ref["dedup"].sum())
    tok = ss.ss_token[:n_ss].long()
    step = 1 << 15
    for r0 in range(0, n_ss, step):
        r1 = min(n_ss, r0 + step)
        assert torch.equal(ss.send_ss[r0:r1].view(torch.int16),
                           b.x.index_select(0, tok[r0:r1]).view(torch.int16)), r0
