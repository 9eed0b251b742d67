"""GPU parity on seeded random problem shapes: every entry point (the
one-call route + assignment + layout against the separate calls), called
through the C ABI, against the CPU oracle on shapes drawn across the whole
documented range (E from 1 to 1024 log-uniform, k up to min(E, 16), R a
divisor of E or any R up to 1024 with a random replica table, rows from one
16-byte chunk to past 1024 chunks, both 16-bit formats, both greedy orders,
fp32 output, logits with many exact ties). The fixed shape lists elsewhere
sit on the kernels' launch-shape boundaries; these land between and across
them in combinations no list names. The bars are those of the other parity
tests: bit-exact indices, counts, offsets and rows, gate weights within rtol
1e-6, the combine and dispatch backward within rtol 4e-3 / atol 1e-3 (fp32
outputs within their accumulation bound)."""
from __future__ import annotations

import os

import numpy as np
import pytest

import synth
from combine_router_topk_amd import binding as B
from pathcheck import say
from test_backward_gpu import run_backward
from test_eplb_gpu import random_table, run_split
from test_fused_plan_gpu import run_both
from test_parity_gpu import run_and_check
from test_fused_single_send_gpu import run_both as run_both_ss
from test_single_send_gpu import check_single_send, run_single_send
from test_stats_gpu import run_stats

import oracle

# The committed sweep: 64 shapes from one seed. MOE_RANDOM_SEED and
# MOE_RANDOM_CASES draw another sweep of any length through the same checks.
DEFAULT_SEED, DEFAULT_CASES = 20_261_203, 64
SWEEP_SEED = int(os.environ.get("MOE_RANDOM_SEED", DEFAULT_SEED))
N_CASES = int(os.environ.get("MOE_RANDOM_CASES", DEFAULT_CASES))
ELEMENT_BUDGET = 12_000_000   # T*k*H: the oracle's rows stay at a few seconds
LARGE_BUDGET = 24_000_000     # one case in four: enough rows for the occupancy-capped launches
CHUNK_BANDS = [(1, 64), (65, 128), (129, 256), (257, 512), (513, 1100)]


def draw_problem(i: int, rng: np.random.Generator) -> dict:
    E = int(min(1024, max(1, round(np.exp(rng.uniform(0.0, np.log(1024.0)))))))
    k = int(rng.integers(1, min(E, 16) + 1))
    table = bool(rng.random() < 0.4)
    if table:
        R = int(rng.integers(1, min(1024, 2 * E + 4) + 1))
        maxrep = int(rng.integers(1, min(16, R) + 1))
    else:
        R = int(rng.choice([d for d in range(1, min(E, 1024) + 1) if E % d == 0]))
        maxrep = 0
    lo, hi = CHUNK_BANDS[int(rng.integers(len(CHUNK_BANDS)))]
    H = 8 * int(rng.integers(lo, hi + 1))
    budget = LARGE_BUDGET if i % 4 == 3 else ELEMENT_BUDGET
    T = int(rng.integers(1, max(1, min(4000, budget // (k * H))) + 1))
    act = synth.F16 if rng.random() < 0.5 else synth.BF16
    bias = str(rng.choice(["none", "zipf1.2", "zipf1.0_perm"] + (["cluster_pairs"] if E >= 2 else [])))
    return dict(i=i, T=T, E=E, k=k, R=R, H=H, act=act, bias=bias, maxrep=maxrep,
                out_f32=bool(rng.random() < 0.3), id_order=bool(table and rng.random() < 0.4),
                ties=bool(rng.random() < 0.3), seed=int(rng.integers(1 << 30)))


def problems(n: int, seed: int) -> list[dict]:
    rng = np.random.default_rng(seed)
    return [draw_problem(i, rng) for i in range(n)]


DEFAULT_PROBLEMS = problems(DEFAULT_CASES, DEFAULT_SEED)
PROBLEMS = problems(N_CASES, SWEEP_SEED)


def case_id(c: dict) -> str:
    rep = f"_rep{c['maxrep']}" if c["maxrep"] else ""
    return f"p{c['i']}_T{c['T']}_E{c['E']}_k{c['k']}_H{c['H']}_R{c['R']}{rep}"


def inputs(c: dict):
    w = synth.Workload(case_id(c), c["T"], c["E"], c["k"], c["H"], c["R"], c["act"], c["bias"], False)
    logits = synth.make_logits(w, c["seed"] % 1000)
    if c["ties"]:
        # a coarse grid: most tokens hold several exactly equal logits
        logits = (np.round(logits * 2.0) / 2.0).astype(np.float32)
    rep = random_table(c["seed"], c["E"], c["R"], c["maxrep"], holes=True) if c["maxrep"] else None
    flags = (B.MOE_FLAG_OUT_F32 if c["out_f32"] else 0) | (B.MOE_FLAG_GREEDY_ID_ORDER if c["id_order"] else 0)
    order = "id" if c["id_order"] else "constrained"
    return w, logits, rep, flags, order


def test_problem_draws_cover_every_band():
    """The committed draws reach every row-width band, both formats, replica
    tables, E past 128, and some batches large enough for the capped launches."""
    P = DEFAULT_PROBLEMS
    bands = {next(j for j, (lo, hi) in enumerate(CHUNK_BANDS) if lo <= c["H"] // 8 <= hi) for c in P}
    assert bands == set(range(len(CHUNK_BANDS)))
    assert {c["act"] for c in P} == {synth.F16, synth.BF16}
    assert any(c["maxrep"] for c in P) and any(not c["maxrep"] for c in P)
    assert any(c["E"] > 128 for c in P) and any(c["E"] <= 16 for c in P)
    assert any(c["T"] * c["k"] >= 4096 and c["H"] > 1024 for c in P)


@pytest.mark.gpu
@pytest.mark.parametrize("c", PROBLEMS, ids=case_id)
def test_random_problem_every_entry_point(c):
    w, logits, rep, flags, order = inputs(c)
    say(f"[case] random {case_id(c)} act={w.dtype_name} bias={c['bias']} ties={c['ties']} "
        f"flags={flags} seed={c['seed']}")
    x = synth.make_x(w, c["seed"] % 1000)
    # forward: route, assign, layout, dispatch, stand-in, combine
    run_and_check(w, flags=flags, rep=rep, order=order, logits=logits, x=x)
    # route, assign and layout as one call: equal to the separate calls
    run_both(w, rep=rep, order=order, logits=logits)
    # and with the single-send rows
    run_both_ss(w, rep=rep, order=order, logits=logits)
    # single-send layout, dispatch and fan-out
    b, ss, expanded = run_single_send(w, logits, x, rep, flags)
    ref = oracle.route_and_layout(w.T, w.E, w.k, w.R, logits, rep, order)
    check_single_send(w, b, ss, expanded, ref)
    # routing statistics and the token-balanced split on the same routing
    run_stats(w, rep=rep, order=order, flags=flags, logits=logits)
    run_split(w, rep=rep, order=order, flags=flags, logits=logits)
    # backward of combine and dispatch (its runner takes the contiguous
    # partition, so only where R divides E)
    if rep is None:
        run_backward(w, c["seed"] % 1000, flags=flags & B.MOE_FLAG_OUT_F32)
