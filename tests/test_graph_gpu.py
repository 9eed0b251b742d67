"""The whole routing path recorded as one HIP graph and replayed: every
replay, with eager work and synchronisations between replays, must give the
outputs of the eager pass bit for bit; a new batch copied into the graph's
input buffers must give the oracle's outputs for that batch."""
import numpy as np
import pytest
import torch

import oracle
import synth
from combine_router_topk_amd import path as P
from pathcheck import bits_to_tensor, check_meta, check_rows, run_gpu, say

pytestmark = pytest.mark.gpu

KEYS = ("idx", "w", "counts", "assign", "active", "rank_of", "expert_offsets", "rank_offsets",
        "pos", "src", "dedup", "send", "y", "out")


def snapshot(b):
    return {k: getattr(b, k).clone() for k in KEYS}


def same_bits(a, b):
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


@pytest.mark.parametrize("w", [synth.TINY, synth.DECODE, synth.scaled(synth.TRAIN_TOP6, T=1500, H=256)],
                         ids=lambda w: w.name)
def test_graph_replays_match_eager(w):
    say(f"[case] graph {w.name}")
    logits, x = synth.make_logits(w, 0), synth.make_x(w, 0)
    rep = synth.replica_table(w)
    b = run_gpu(w, logits, x, rep)            # eager pass
    want = snapshot(b)
    g = P.capture(b)
    torch.cuda.synchronize()
    for r in range(3):
        for k in ("send", "y", "out", "w"):   # eager work between replays
            getattr(b, k).fill_(float("nan"))
        b.pos.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in KEYS:
            assert same_bits(getattr(b, k), want[k]), (r, k)

    # a new batch in the same buffers
    logits2, x2 = synth.make_logits(w, 7), synth.make_x(w, 7)
    b.logits.copy_(torch.from_numpy(logits2))
    b.x.copy_(bits_to_tensor(x2, w.act_dtype))
    g.replay()
    torch.cuda.synchronize()
    ref = oracle.route_and_layout(w.T, w.E, w.k, w.R, logits2, rep)
    check_meta(b, ref, w.T, w.k)
    rng = np.random.default_rng(3)
    rows = np.unique(rng.choice(w.T * w.k, size=min(256, w.T * w.k), replace=False))
    toks = np.unique(rng.choice(w.T, size=min(128, w.T), replace=False))
    check_rows(b, ref, x2, w, rows, toks, out_f32=False)


@pytest.mark.parametrize("w", [synth.DECODE, synth.scaled(synth.TRAIN_TOP2, T=2000, H=512)],
                         ids=lambda w: w.name)
def test_graph_of_every_entry_point(w):
    """The forward pass, the single-send layout, dispatch and fan-out, the
    backward of combine and dispatch, the routing statistics (cleared by a
    fill kernel, not a memset), the token-balanced split and the one-call
    route + assignment + layout (with and without the single-send rows),
    all recorded in one graph: three replays, with the outputs overwritten between them,
    each equal bit for bit to the eager pass."""
    from combine_router_topk_amd import binding as B
    say(f"[case] graph of every entry point {w.name}")
    logits, x = synth.make_logits(w, 0), synth.make_x(w, 0)
    rep = synth.replica_table(w)
    b = run_gpu(w, logits, x, rep)
    ss = P.allocate_single_send(b)
    st = P.allocate_stats(b)
    sp = P.allocate_split(b)
    dout = bits_to_tensor(synth.make_grad(w, 0, w.T), w.act_dtype).to(b.x.device)
    dy = torch.empty_like(b.y)
    dw = torch.empty(w.T * w.k, dtype=torch.float32, device=b.x.device)
    dx = torch.empty_like(b.x)
    send_fwd = b.send.clone()
    steps = P.STEPS + (
        lambda b_: P.layout_single_send(b_, ss),
        lambda b_: P.single_send_dispatch(b_, ss),
        lambda b_: P.single_send_expand(b_, ss),
        lambda b_: B.moe_combine_backward(b_.p, dout, b_.y, b_.pos, b_.w, dy, dw),
        lambda b_: B.moe_dispatch_backward(b_.p, dy, b_.pos, dx),
        lambda b_: P.routing_stats(b_, st),
        lambda b_: P.token_balanced_split(b_, sp),
        P.route_assign_layout,  # rewrites the routing outputs with the same values
        lambda b_: P.route_assign_layout_single_send(b_, ss),  # and the single-send rows
    )
    for step in steps[len(P.STEPS):]:
        step(b)
    torch.cuda.synchronize()
    outs = {**{k: getattr(b, k) for k in KEYS},
            "ss_rank_offsets": ss.ss_rank_offsets, "ss_row": ss.ss_row, "send_ss": ss.send_ss,
            "dy": dy, "dw": dw, "dx": dx, "send_counts": st.send_counts, "coselect": st.coselect,
            "stats": st.stats, "gpu_of_pair": sp.gpu_of_pair, "split_active": sp.active,
            "split_tokens": sp.tokens}
    n_ss = int(ss.ss_rank_offsets[-1])
    want = {k: (v[:n_ss] if k == "send_ss" else v).clone() for k, v in outs.items()}
    assert torch.equal(b.send.view(torch.int16), send_fwd.view(torch.int16))  # fan-out == dispatch
    g = P.capture(b, steps)
    torch.cuda.synchronize()
    for r in range(3):
        for t in outs.values():               # eager work between replays
            if t.dtype.is_floating_point:
                t.fill_(float("nan"))
            else:
                t.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in outs.items():
            got = v[:n_ss] if k == "send_ss" else v
            assert same_bits(got, want[k]), (r, k)
