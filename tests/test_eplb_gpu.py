"""GPU parity of the token-balanced (EPLB-style) split against the CPU oracle,
through the C ABI, on the route and layout the GPU wrote (checked against the
oracle first): the GPU of every pair, the activated replicas and the pairs
served per GPU, all bit-exact; plus the decode-table closed form (36 activated
experts per GPU under token balance, 32 under the greedy)."""
import json

import numpy as np
import pytest
import torch

import oracle
import synth
from combine_router_topk_amd import binding as B
from combine_router_topk_amd import path as P
from pathcheck import check_meta, host, run_gpu, say

pytestmark = pytest.mark.gpu


def run_split(w, seed=0, rep="table", order="constrained", flags=0, logits=None):
    say(f"[case] token-balanced split {w.name} seed={seed}")
    logits = synth.make_logits(w, seed) if logits is None else logits
    rep = synth.replica_table(w) if isinstance(rep, str) else rep
    x = synth.make_x(synth.scaled(w, H=8), seed)
    ref = oracle.route_and_layout(w.T, w.E, w.k, w.R, logits, rep, order)
    b = run_gpu(synth.scaled(w, H=8), logits, x, rep, flags)
    check_meta(b, ref, w.T, w.k)
    sp = P.allocate_split(b)
    sp.gpu_of_pair.fill_(-9)
    P.token_balanced_split(b, sp)
    torch.cuda.synchronize()
    want = oracle.token_balanced_split(ref["idx"], ref["counts"], ref["pos"],
                                       ref["expert_offsets"], w.R, rep)
    assert np.array_equal(host(sp.gpu_of_pair), want), "gpu_of_pair"
    act = oracle.token_balanced_activations(ref["counts"], w.R, rep)
    tok = oracle.split_tokens_per_gpu(ref["counts"], w.R, rep)
    assert host(sp.active).tolist() == act.tolist(), "active"
    assert host(sp.tokens).tolist() == tok.tolist(), "tokens"
    say(f"  max activated: greedy {int(ref['active'].max())}, token balance {int(act.max())}; "
        f"max pairs per GPU: greedy {int(np.diff(ref['rank_offsets']).max())}, "
        f"token balance {int(tok.max())}")
    return b, sp, ref


def random_table(seed, E, R, maxrep, holes=False):
    rng = np.random.default_rng(seed)
    rep = np.full((E, maxrep), -1, np.int32)
    for e in range(E):
        n = int(rng.integers(1, min(maxrep, R) + 1))
        rep[e, :n] = rng.choice(R, size=n, replace=False)
        if holes and n < maxrep:
            # -1 entries between valid ones; column 0 stays the (valid) primary
            rep[e, 1:] = rng.permutation(rep[e, 1:])
    return rep


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_split_decode(seed):
    run_split(synth.DECODE, seed)


def test_split_decode_all_active_closed_form():
    """Token t ranks experts 8t .. 8t+7 (mod 256) first: every expert gets
    exactly 8 pairs, so all 256 are active."""
    w = synth.DECODE
    logits = np.zeros((w.T, w.E), np.float32)
    for j in range(w.k):
        logits[np.arange(w.T), (np.arange(w.T) * w.k + j) % w.E] = 10.0 - j
    b, sp, ref = run_split(w, 0, logits=logits)
    assert (ref["counts"] == 8).all()
    assert host(sp.active).tolist() == [36] * 8
    assert host(b.active).tolist() == [32] * 8
    assert host(sp.tokens).tolist() == [256] * 8


@pytest.mark.parametrize("maxrep,holes", [(2, False), (3, True), (4, False), (16, True)])
def test_split_random_tables(maxrep, holes):
    E, R = 64, 8
    rep = random_table(40 + maxrep, E, R, maxrep, holes)
    w = synth.Workload(f"split_rep{maxrep}", 1500, E, 6, 8, R, synth.BF16, "zipf1.2", False)
    run_split(w, 2, rep=rep)


def test_split_id_order_and_no_table():
    rep = random_table(77, 32, 4, 3)
    w = synth.Workload("split_id", 700, 32, 4, 8, 4, synth.F16, "none", False)
    run_split(w, 1, rep=rep, order="id", flags=B.MOE_FLAG_GREEDY_ID_ORDER)
    run_split(synth.scaled(synth.TRAIN_TOP2, T=2000), 0)   # one copy per expert


@pytest.mark.parametrize("w", [synth.DECODE, synth.TRAIN_TOP6, synth.LARGE], ids=lambda w: w.name)
def test_split_full_size(w):
    run_split(w, 0)


def test_split_edge_shapes_and_empty():
    run_split(synth.Workload("split_E1", 20, 1, 1, 8, 1, synth.BF16, "none", False), 0)
    rep = random_table(5, 1024, 1024, 4)
    run_split(synth.Workload("split_E1024", 300, 1024, 16, 8, 1024, synth.BF16, "none", False), 0,
              rep=rep)
    w = synth.Workload("split_empty", 0, 8, 2, 8, 4, synth.F16, "none", False)
    say("[case] token-balanced split, empty batch")
    b = run_gpu(w, np.zeros((0, 8), np.float32), np.zeros((0, 8), np.uint16), None)
    sp = P.allocate_split(b)
    P.token_balanced_split(b, sp)
    torch.cuda.synchronize()
    assert host(sp.active).tolist() == [0] * 4 and host(sp.tokens).tolist() == [0] * 4


def test_routing_record_matches_the_oracle():
    """path.record on the replicated decode workload: per-rank send bytes,
    the dedup total, activated experts per GPU and the assign map, against
    the oracle; the single-send bytes sum to the dedup rows."""
    w = synth.DECODE
    say("[case] routing record")
    logits, x = synth.make_logits(w, 1), synth.make_x(w, 1)
    rep = synth.replica_table(w)
    ref = oracle.route_and_layout(w.T, w.E, w.k, w.R, logits, rep)
    b = run_gpu(w, logits, x, rep)
    ss = P.allocate_single_send(b)
    P.layout_single_send(b, ss)
    rec = P.record(b, ss)
    rb = w.H * 2
    assert rec["send_bytes"] == (np.diff(ref["rank_offsets"]) * rb).tolist()
    assert sum(rec["send_bytes"]) == w.T * w.k * rb and rec["rows"] == w.T * w.k
    assert rec["dedup_rows"] == int(ref["dedup"].sum())
    assert sum(rec["ss_send_bytes"]) == rec["dedup_rows"] * rb
    assert rec["active_per_gpu"] == ref["active"].tolist()
    assert rec["assign"] == ref["assign"].tolist() and rec["counts"] == ref["counts"].tolist()
    json.dumps(rec)
