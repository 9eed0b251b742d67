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
