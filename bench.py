"""Benchmark of the single-GPU MoE routing path on MI355X.

One step = one pass of the whole path over one batch resident in HBM:
the one-call plan (route: top-k, gate weights, demand vector; greedy
replica assignment; layout: offsets, permutation, dedup) -> dispatch ->
expert stand-in -> combine. The headline is dispatch+combine GB/s of algorithmic bytes,
2 (1 + k) T H b, over the two kernels' HIP-event durations (events without
the system-scope fence, see timing_event_type), and routed rows/s
(T k rows over the same time). By default the 256 MB Infinity Cache and the L2s
are flushed (a 1 GiB fill) before the dispatch and before the combine, outside
their event brackets, so both read from HBM.

After the headline loop, and outside it, every other workload is measured
the same way (`workloads`), the same batch also times the route, assignment
and layout as separate calls, the single-send variant (layout,
one-row-per-rank dispatch, receiver fan-out), the backward of the dispatch
and the combine, and the routing statistics, and the replicated decode
workload compares the greedy replica assignment with token-balanced routing
and times a decode step eager against a HIP graph replay; each is reported in
its own object of the JSON line. Before any of it, and before the GPU is
touched, the CPU oracle is timed on one core and on every usable host core
(`cpu_baseline`).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "dispatch+combine HBM GB/s (% of peak) and routed rows/s at T=16384,E=64,top-2"
PEAK_GBPS = 8000.0          # MI355X HBM3E peak
DEFAULT_WORKLOAD = "train_T16384_E64_k2_H4096_bf16_clustered"
PROFILE_MD = os.path.join(ROOT, "profiles", "dispatch_combine_T16384_E64_k2_H4096_bf16.md")
FLUSH_BYTES = 1 << 30


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=int(os.environ.get("WORLD_SIZE", "1")))
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--warm-cache", action="store_true", help="no cache flush before dispatch/combine")
    ap.add_argument("--warm-steps", type=int, default=20,
                    help="timed dispatch+combine passes without the cache flush, reported beside the headline (0 = skip)")
    ap.add_argument("--single-send-steps", type=int, default=20,
                    help="timed passes of the single-send variant after the headline loop (0 = skip)")
    ap.add_argument("--backward-steps", type=int, default=20,
                    help="timed passes of the dispatch/combine backward after the headline loop (0 = skip)")
    ap.add_argument("--stats-steps", type=int, default=20,
                    help="timed calls of the routing statistics after the headline loop (0 = skip)")
    ap.add_argument("--eplb-steps", type=int, default=20,
                    help="timed token-balanced splits on the replicated decode workload (0 = skip)")
    ap.add_argument("--graph-steps", type=int, default=200,
                    help="decode steps timed eager and as a HIP graph replay (0 = skip)")
    ap.add_argument("--workload-steps", type=int, default=10,
                    help="timed passes of every other workload, reported in `workloads` (0 = skip)")
    ap.add_argument("--cpu-tokens", type=int, default=1 << 30,
                    help="tokens in the oracle's CPU-baseline sample (0 = skip; default all)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="repeat the oracle's timed stages until this much CPU time is spent")
    return ap.parse_args()


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    with open(os.path.join(ROOT, "combine_router_topk_amd", "csrc", "rows.hip"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def row_kernel_names(T: int, k: int, H: int):
    """Names of the dispatch and combine kernels that launches of this shape
    run, for the roofline entries. They follow the launch rules of the
    library's row kernels: 128-chunk row slices for dispatch rows over 512
    chunks in launches of at least 4096 slices, or of 257-512 chunks with
    k >= 5 in launches of at least 16384, and for combine rows over 256
    chunks with k >= 5 in launches of at least 12288."""
    cpr = H // 8
    slices = T * -(-cpr // 128)
    sliced_d = (cpr > 512 and slices >= 4096) or (cpr > 256 and k >= 5 and slices >= 16384)
    d = "dispatch_slice_kernel" if sliced_d else "dispatch_kernel"
    c = "combine_slice_kernel" if cpr > 256 and k >= 5 and slices >= 12288 else "combine_kernel"
    return d, c


def traffic_from_profiles(kernel: str, workload: str):
    """HBM bytes per launch measured with rocprofv3 PMC counters, if the
    counters were taken on the current kernel source for this workload."""
    try:
        with open(PROFILE_MD) as f:
            line = next(l for l in f if l.startswith("traffic-json: "))
        rec = json.loads(line[len("traffic-json: "):])
    except (OSError, ValueError, StopIteration):
        return None
    if rec.get("rows_hip_sha") != kernel_source_digest() or rec.get("workload") != workload:
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


def timing_event_type(lib, torch):
    """HIP timing events with the interface of torch.cuda.Event(enable_timing=
    True), taken from the HIP runtime the routing library launches with (its
    handle resolves the runtime's symbols) and recorded on torch's current
    stream, which is the stream the library's kernels run on. They are created
    with hipEventDisableSystemFence: recording one then skips the system-scope
    cache writeback and invalidation, which the HIP headers name as the more
    accurate choice for events used only to time work. Elapsed times are read
    after a device synchronisation."""
    import ctypes
    vp = ctypes.c_void_p
    create, record = lib.hipEventCreateWithFlags, lib.hipEventRecord
    elapsed, destroy = lib.hipEventElapsedTime, lib.hipEventDestroy
    create.argtypes, create.restype = [ctypes.POINTER(vp), ctypes.c_uint], ctypes.c_int
    record.argtypes, record.restype = [vp, vp], ctypes.c_int
    elapsed.argtypes, elapsed.restype = [ctypes.POINTER(ctypes.c_float), vp, vp], ctypes.c_int
    destroy.argtypes, destroy.restype = [vp], ctypes.c_int
    disable_system_fence = 0x20000000

    class Event:
        def __init__(self):
            self.h = vp()
            if create(ctypes.byref(self.h), disable_system_fence) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")

        def record(self):
            if record(self.h, vp(torch.cuda.current_stream().cuda_stream)) != 0:
                raise RuntimeError("hipEventRecord failed")

        def elapsed_time(self, end) -> float:
            ms = ctypes.c_float()
            if elapsed(ctypes.byref(ms), self.h, end.h) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            return ms.value

        def __del__(self):
            if self.h:
                destroy(self.h)

    return Event


def cpu_baseline(w, seed: int, tokens: int, min_seconds: float):
    """The oracle, as it stands, on the first `tokens` tokens of the same
    workload: its dispatch and combine timed on the host (repeated until
    `min_seconds` have been spent, at least once), in the metric's unit.
    numpy runs these element-wise steps on one thread."""
    import numpy as np

    import oracle
    import synth

    sub = synth.scaled(w, T=min(tokens, w.T))
    logits = synth.make_logits(w, seed)[:sub.T]
    x = synth.make_x(w, seed)[:sub.T]
    rep = synth.replica_table(w)
    meta = oracle.route_and_layout(sub.T, sub.E, sub.k, sub.R, logits, rep)
    secs, reps = 0.0, 0
    while reps == 0 or secs < min_seconds:
        t0 = time.perf_counter()
        send = oracle.dispatch(x, meta["pos"], sub.k)
        t1 = time.perf_counter()
        y = oracle.expert_standin(send, meta["idx"].ravel()[meta["src"]], sub.E, sub.act_dtype)
        t2 = time.perf_counter()
        oracle.combine(y, meta["pos"], meta["w"], sub.k, sub.act_dtype)
        t3 = time.perf_counter()
        secs += (t1 - t0) + (t3 - t2)
        reps += 1
        del send, y
    nbytes = sub.dispatch_combine_bytes() * reps
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), None)
    except OSError:
        pass
    return {"value": round(nbytes / secs / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "host_cpu": cpu_model, "host_threads": os.cpu_count(),
            "sample": f"first {sub.T} of {w.T} tokens of {w.name}, {reps} passes; oracle dispatch + "
                      f"fp64 combine ({secs:.2f} s for {nbytes} algorithmic bytes)",
            "routed_rows_per_s": round(reps * sub.T * sub.k / secs, 1)}


def host_cores() -> int:
    """Host threads this process may use, at most 16 (one GPU's share of the
    host on the GPU machines)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


_ALL = {}  # the batch the forked workers of cpu_baseline_all_cores read


def chunk_layout(pos_all, idx, k: int, t0: int, t1: int):
    """Send layout of tokens [t0, t1) alone: their pairs in the order they
    have in the whole batch's send buffer, renumbered from 0 (pos), and the
    expert of each of those rows."""
    import numpy as np
    pos_full = pos_all[t0 * k:t1 * k]
    pos = np.empty_like(pos_full)
    pos[np.argsort(pos_full, kind="stable")] = np.arange(pos_full.shape[0], dtype=pos.dtype)
    src = np.empty_like(pos)
    src[pos] = np.arange(pos.shape[0], dtype=pos.dtype)
    return pos, idx[t0:t1].ravel()[src]


def _oracle_chunk_worker(args):
    """One worker of the all-cores leg: the oracle's dispatch and combine on
    its own contiguous token chunk, repeated until min_seconds have passed;
    returns (algorithmic bytes moved, seconds)."""
    import oracle
    t0, t1, min_seconds = args
    d = _ALL
    k, H = d["k"], d["H"]
    x = d["x"][t0:t1]
    pos, row_e = chunk_layout(d["pos"], d["idx"], k, t0, t1)
    w = d["w"][t0:t1]
    secs, reps = 0.0, 0
    while reps == 0 or secs < min_seconds:
        a = time.perf_counter()
        send = oracle.dispatch(x, pos, k)
        b = time.perf_counter()
        y = oracle.expert_standin(send, row_e, d["E"], d["act"])
        c = time.perf_counter()
        oracle.combine(y, pos, w, k, d["act"])
        e = time.perf_counter()
        secs += (b - a) + (e - c)
        reps += 1
    return 2 * (1 + k) * (t1 - t0) * H * 2 * reps, secs


def cpu_baseline_all_cores(w, seed: int, min_seconds: float) -> dict:
    """The oracle, as it stands, on every usable host core at once: the batch
    cut into one contiguous token chunk per core, each chunk's dispatch and
    combine run by the oracle in its own process (forked before anything
    touches the GPU), no new arithmetic. Rate = total algorithmic bytes over
    the longest worker's timed seconds."""
    import multiprocessing as mp

    import oracle
    import synth

    logits, x = synth.make_logits(w, seed), synth.make_x(w, seed)
    meta = oracle.route_and_layout(w.T, w.E, w.k, w.R, logits, synth.replica_table(w))
    _ALL.update(x=x, pos=meta["pos"], idx=meta["idx"], w=meta["w"], k=w.k, H=w.H, E=w.E,
                act=w.act_dtype)
    n = host_cores()
    bounds = [(w.T * i // n, w.T * (i + 1) // n, min_seconds) for i in range(n)]
    with mp.get_context("fork").Pool(n) as pool:
        res = pool.map(_oracle_chunk_worker, bounds)
    _ALL.clear()
    nbytes = sum(r[0] for r in res)
    secs = max(r[1] for r in res)
    return {"value": round(nbytes / secs / 1e9, 3), "unit": "GB/s", "cores": n, "kind": "oracle",
            "sample": f"all {w.T} tokens of {w.name} in {n} contiguous chunks, one process per core, "
                      f"each repeating the oracle's dispatch + fp64 combine for at least {min_seconds:.0f} s",
            "routed_rows_per_s": round(nbytes / (2 * (1 + w.k) * w.H * 2) * w.k / secs, 1)}


def cpu_next_rows(w, seed: int, tokens: int, min_seconds: float):
    """The oracle, as it stands, on the rows beyond dispatch+combine, on the
    same token sample as the dispatch+combine baseline, each step repeated
    until `min_seconds` of host time (at least once), in the units of the GPU
    legs: the single-send layout in ms, the single-send dispatch and fan-out
    and the two backward kernels in GB/s of algorithmic bytes, the routing
    statistics in pairs per second; the token-balanced split on the
    replicated decode workload, as on the GPU, in pairs per second."""
    import numpy as np

    import oracle
    import synth

    def timed(fn):
        secs, n, out = 0.0, 0, None
        while n == 0 or secs < min_seconds:
            t0 = time.perf_counter()
            out = fn()
            secs += time.perf_counter() - t0
            n += 1
        return secs / n, out

    sub = synth.scaled(w, T=min(tokens, w.T))
    T, k, act, rb = sub.T, sub.k, sub.act_dtype, sub.H * 2
    x = synth.make_x(w, seed)[:T]
    m = oracle.route_and_layout(T, sub.E, k, sub.R, synth.make_logits(w, seed)[:T],
                                synth.replica_table(w))
    lay_s, (ss_off, ss_row, ss_tok) = timed(
        lambda: oracle.single_send_layout(m["idx"], m["rank_of"], sub.R))
    n_ss = int(ss_off[-1])
    dsp_s, send_ss = timed(lambda: oracle.single_send_dispatch(x, ss_tok))
    exp_s, _ = timed(lambda: oracle.single_send_expand(send_ss, ss_row, m["src"]))
    del send_ss
    y = oracle.expert_standin(oracle.dispatch(x, m["pos"], k), m["idx"].ravel()[m["src"]], sub.E, act)
    dout = synth.make_grad(w, seed, T)

    def combine_backward():
        dy = oracle.combine_backward_dy(dout, m["src"], m["w"], k, act)
        oracle.combine_backward_dw(y, dout, m["pos"], k, act)
        return dy

    cb_s, dy = timed(combine_backward)
    db_s, _ = timed(lambda: oracle.dispatch_backward(dy, m["pos"], k, act))
    del y, dy
    st_s, _ = timed(lambda: oracle.routing_stats(m["idx"], m["counts"], m["rank_of"], sub.E, sub.R))
    d = synth.DECODE
    drep = synth.replica_table(d)
    md = oracle.route_and_layout(d.T, d.E, d.k, d.R, synth.make_logits(d, seed), drep)
    sp_s, _ = timed(lambda: oracle.token_balanced_split(md["idx"], md["counts"], md["pos"],
                                                        md["expert_offsets"], d.R, drep))
    gbps = lambda nbytes, secs: round(nbytes / secs / 1e9, 3)
    return {"sample": f"first {T} of {w.T} tokens of {w.name}; the split on {d.name}",
            "single_send": {"layout_ms": round(lay_s * 1e3, 3),
                            "dispatch_GBps": gbps((T + n_ss) * rb, dsp_s),
                            "expand_GBps": gbps((n_ss + T * k) * rb, exp_s)},
            "backward": {"combine_backward_GBps": gbps((1 + 2 * k) * T * rb, cb_s),
                         "dispatch_backward_GBps": gbps((1 + k) * T * rb, db_s)},
            "routing_stats_pairs_per_s": round(T * k / st_s, 1),
            "token_balanced_split_pairs_per_s": round(d.T * d.k / sp_s, 1)}


def warm_leg(P, b, steps, ev, np, torch, dc_bytes):
    """Dispatch and combine back to back without the cache flush: the inputs
    may then come partly from the 256 MB Infinity Cache, so this is reported
    beside the cold headline, never as it."""
    marks = []
    for i in range(steps + 3):
        e = [ev() for _ in range(4)]
        e[0].record()
        P.dispatch(b)
        e[1].record()
        P.standin(b)
        e[2].record()
        P.combine(b)
        e[3].record()
        if i >= 3:
            marks.append(e)
    torch.cuda.synchronize()
    d = float(np.mean([m[0].elapsed_time(m[1]) for m in marks]))
    c = float(np.mean([m[2].elapsed_time(m[3]) for m in marks]))
    return {"steps": steps, "stage_ms": {"dispatch": round(d, 4), "combine": round(c, 4)},
            "GBps": round(dc_bytes / ((d + c) / 1e3) / 1e9, 1)}


def single_send_leg(P, w, b, flush, steps, ev, np, torch):
    """The single-send variant on the same batch, timed after the headline
    loop: route, assignment and single-send layout in one call
    (`one_call_plan`), the single-send layout call alone (the plain layout
    plus the single-send rows), the dispatch of one row per (token,
    destination rank), and the receiver fan-out back to the expert-grouped
    buffer, each cold-cache like the headline. Algorithmic bytes: dispatch (T + n_ss) H b, fan-out
    (n_ss + T k) H b (each single-send row read once, every expert row
    written once)."""
    ss = P.allocate_single_send(b)
    marks, plan_marks = [], []
    for i in range(steps + 2):
        # route, assignment and single-send layout in one call, enqueued
        # behind a flush so the bracket holds kernel time
        if flush is not None:
            flush.fill_(14.0)
        p0, p1 = ev(), ev()
        p0.record()
        P.route_assign_layout_single_send(b, ss)
        p1.record()
        e = [ev() for _ in range(6)]
        e[0].record()
        P.layout_single_send(b, ss)
        e[1].record()
        if flush is not None:
            flush.fill_(4.0)
        e[2].record()
        P.single_send_dispatch(b, ss)
        e[3].record()
        if flush is not None:
            flush.fill_(5.0)
        e[4].record()
        P.single_send_expand(b, ss)
        e[5].record()
        if i >= 2:
            marks.append(e)
            plan_marks.append((p0, p1))
    torch.cuda.synchronize()
    avg = lambda i: float(np.mean([m[i].elapsed_time(m[i + 1]) for m in marks]))
    lay_ms, dsp_ms, exp_ms = avg(0), avg(2), avg(4)
    plan_ms = float(np.mean([a.elapsed_time(c) for a, c in plan_marks]))
    n_ss = int(ss.ss_rank_offsets[-1].item())
    rb = w.H * 2
    d_bytes = (w.T + n_ss) * rb
    x_bytes = (n_ss + w.T * w.k) * rb
    return {"rows": n_ss, "raw_rows": w.T * w.k, "rows_cut_frac": round(1 - n_ss / (w.T * w.k), 4),
            "steps": steps,
            "stage_ms": {"one_call_plan": round(plan_ms, 4), "layout": round(lay_ms, 4),
                         "dispatch": round(dsp_ms, 4), "expand": round(exp_ms, 4)},
            "dispatch_GBps": round(d_bytes / (dsp_ms / 1e3) / 1e9, 1),
            "expand_GBps": round(x_bytes / (exp_ms / 1e3) / 1e9, 1),
            "dispatch_bytes": d_bytes, "expand_bytes": x_bytes}


def backward_leg(B, w, b, flush, steps, ev, np, torch, synth, seed):
    """The backward of the combine (dy and dw in one kernel) and of the
    dispatch (dx) on the same batch, each cold-cache, timed after the
    headline loop. Algorithmic bytes: combine backward (1 + 2k) T H b (dout
    read once, y read and dy written per slot), dispatch backward
    (1 + k) T H b; the 4-8 bytes per slot of pos, w and dw are left out, as in
    the forward."""
    dout = synth.make_grad(w, seed, w.T)
    tdt = b.x.dtype
    g = torch.from_numpy(dout.view(np.int16)).view(tdt).to(b.x.device)
    dy = torch.empty_like(b.y)
    dw = torch.empty(w.T * w.k, dtype=torch.float32, device=b.x.device)
    dx = torch.empty_like(b.x)
    marks = []
    for i in range(steps + 2):
        e = [ev() for _ in range(4)]
        if flush is not None:
            flush.fill_(6.0)
        e[0].record()
        B.moe_combine_backward(b.p, g, b.y, b.pos, b.w, dy, dw)
        e[1].record()
        if flush is not None:
            flush.fill_(7.0)
        e[2].record()
        B.moe_dispatch_backward(b.p, dy, b.pos, dx)
        e[3].record()
        if i >= 2:
            marks.append(e)
    torch.cuda.synchronize()
    cb_ms = float(np.mean([m[0].elapsed_time(m[1]) for m in marks]))
    db_ms = float(np.mean([m[2].elapsed_time(m[3]) for m in marks]))
    rb = w.H * 2
    cb_bytes = (1 + 2 * w.k) * w.T * rb
    db_bytes = (1 + w.k) * w.T * rb
    return {"steps": steps,
            "stage_ms": {"combine_backward": round(cb_ms, 4), "dispatch_backward": round(db_ms, 4)},
            "combine_backward_GBps": round(cb_bytes / (cb_ms / 1e3) / 1e9, 1),
            "dispatch_backward_GBps": round(db_bytes / (db_ms / 1e3) / 1e9, 1),
            "combine_backward_bytes": cb_bytes, "dispatch_backward_bytes": db_bytes}


def stats_leg(P, w, b, flush, steps, ev, np, torch):
    """Routing statistics of the batch (send-counts matrix, co-selection
    histogram, max/mean, Gini, Dirichlet alpha, locality), timed over
    `steps` calls; plus the share of the tokens' expert pairs held by the
    most frequent 0.8% of pairs, read from the co-selection histogram. A fill
    of the flush buffer before each call keeps the GPU busy while the host
    enqueues the call's three launches, so the bracket holds kernel time,
    not launch latency (and the inputs come from HBM)."""
    st = P.allocate_stats(b)
    marks = []
    for i in range(steps + 2):
        if flush is not None:
            flush.fill_(12.0)
        a, c = ev(), ev()
        a.record()
        P.routing_stats(b, st)
        c.record()
        if i >= 2:
            marks.append((a, c))
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(c) for a, c in marks]))
    vals = st.stats.cpu().numpy()
    C = st.coselect.cpu().numpy().astype(np.int64)
    E = w.E
    iu = np.triu_indices(E, 1)
    pairs = np.sort(C[iu])[::-1]
    top = int(np.ceil(0.008 * pairs.shape[0]))
    cover = float(pairs[:top].sum()) / max(1, int(pairs.sum()))
    f = lambda v: None if not np.isfinite(v) else round(float(v), 6)
    return {"steps": steps, "ms": round(ms, 4), "pairs_per_s": round(w.T * w.k / (ms / 1e3), 1),
            "max_over_mean": f(vals[0]), "gini": f(vals[1]),
            "dirichlet_alpha": f(vals[2]), "locality": f(vals[3]),
            "top_0.8pct_pairs_share": round(cover, 4)}


def eplb_leg(P, B, synth, np, torch, dev, flush, steps, ev, seed):
    """The greedy replica assignment against token-balanced (EPLB-style)
    routing on the replicated decode workload (the one workload with
    replicas): maximum activated experts and maximum pairs per GPU under
    each, and the time of the token-balanced split (its two launches
    enqueued behind a fill of the flush buffer, as in stats_leg)."""
    w = synth.DECODE
    logits, x = synth.make_logits(w, seed), synth.make_x(w, seed)
    rep = synth.replica_table(w)
    tdt = torch.float16 if w.act_dtype == synth.F16 else torch.bfloat16
    p = B.make_problem(w.T, w.E, w.k, w.H, w.R, w.act_dtype)
    b = P.allocate(p, torch.from_numpy(logits), torch.from_numpy(x.view(np.int16)).view(tdt),
                   torch.from_numpy(rep), device=dev)
    P.route(b)
    P.assign(b)
    P.layout(b)
    sp = P.allocate_split(b)
    marks = []
    for i in range(steps + 2):
        if flush is not None:
            flush.fill_(13.0)
        a, c = ev(), ev()
        a.record()
        P.token_balanced_split(b, sp)
        c.record()
        if i >= 2:
            marks.append((a, c))
    torch.cuda.synchronize()
    g_act = int(b.active.max().item())
    e_act = int(sp.active.max().item())
    g_tok = int((b.rank_offsets[1:] - b.rank_offsets[:-1]).max().item())
    e_tok = int(sp.tokens.max().item())
    ms = float(np.mean([a.elapsed_time(c) for a, c in marks]))
    rec = P.record(b)
    return {"workload": w.name, "steps": steps, "ms": round(ms, 4),
            "routing_record": {key: rec[key] for key in ("send_bytes", "dedup_rows", "active_per_gpu",
                                                        "assign")},
            "pairs_per_s": round(w.T * w.k / (ms / 1e3), 1),
            "max_activated": {"greedy": g_act, "token_balanced": e_act},
            "greedy_below_token_balanced": round(1 - g_act / e_act, 4) if e_act else None,
            "max_pairs_per_gpu": {"greedy": g_tok, "token_balanced": e_tok}}


def graph_leg(P, B, synth, np, torch, dev, steps, seed):
    """The whole path on the replicated decode workload, where every kernel is
    small and the host's launches set the pace: wall time per step for eager
    calls against one replay of a HIP graph holding the same pass (warm
    cache, the stream drained after each step in both cases), also with
    route, assign and layout as one call (`fused_plan`). `pipelined_us_per_step`
    issues the steps back to back and drains the stream once at the end, as
    a loop over layers does: the device's own time per step once the host's
    launch and synchronisation are off the critical path."""
    w = synth.DECODE
    logits, x = synth.make_logits(w, seed), synth.make_x(w, seed)
    rep = synth.replica_table(w)
    p = B.make_problem(w.T, w.E, w.k, w.H, w.R, w.act_dtype)
    b = P.allocate(p, torch.from_numpy(logits), torch.from_numpy(x.view(np.int16)).view(torch.float16),
                   torch.from_numpy(rep), device=dev)
    g = P.capture(b)
    gf = P.capture(b, P.FUSED_STEPS)
    torch.cuda.synchronize()

    def timed(fn):
        for _ in range(5):
            fn()
            torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
            torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps * 1e6

    def pipelined(fn):
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps * 1e6

    eager_us = timed(lambda: P.run(b))
    graph_us = timed(g.replay)
    fused_eager_us = timed(lambda: [step(b) for step in P.FUSED_STEPS])
    fused_graph_us = timed(gf.replay)
    graph_pipe_us = pipelined(g.replay)
    fused_graph_pipe_us = pipelined(gf.replay)
    return {"workload": w.name, "steps": steps, "eager_us_per_step": round(eager_us, 1),
            "graph_us_per_step": round(graph_us, 1),
            "graph_pipelined_us_per_step": round(graph_pipe_us, 1),
            "fused_plan": {"eager_us_per_step": round(fused_eager_us, 1),
                           "graph_us_per_step": round(fused_graph_us, 1),
                           "graph_pipelined_us_per_step": round(fused_graph_pipe_us, 1)}}


def workloads_leg(P, B, synth, np, torch, dev, flush, ev, seed, steps, skip) -> dict:
    """Every other workload, measured the way the headline is: the one-call
    plan, then dispatch and combine each after a cache flush (cold), HIP
    events on the stream; dispatch+combine GB/s of algorithmic bytes,
    2 (1 + k) T H b, its fraction of peak, routed rows/s, and the roofline of
    the slower of the two kernels. The decode batch is latency-bound: its
    stage times are the figures that matter there."""
    out = {}
    for w in synth.WORKLOADS:
        if w.name == skip:
            continue
        logits, x = synth.make_logits(w, seed), synth.make_x(w, seed)
        rep = synth.replica_table(w)
        tdt = torch.float16 if w.act_dtype == synth.F16 else torch.bfloat16
        p = B.make_problem(w.T, w.E, w.k, w.H, w.R, w.act_dtype)
        b = P.allocate(p, torch.from_numpy(logits), torch.from_numpy(x.view(np.int16)).view(tdt),
                       None if rep is None else torch.from_numpy(rep), device=dev)
        del logits, x
        marks = []
        for i in range(steps + 2):
            e = [ev() for _ in range(6)]
            if flush is not None:
                flush.fill_(9.0)
            e[0].record()
            P.route_assign_layout(b)
            e[1].record()
            if flush is not None:
                flush.fill_(10.0)
            e[2].record()
            P.dispatch(b)
            e[3].record()
            P.standin(b)
            if flush is not None:
                flush.fill_(11.0)
            e[4].record()
            P.combine(b)
            e[5].record()
            if i >= 2:
                marks.append(e)
        torch.cuda.synchronize()
        avg = lambda i: float(np.mean([m[i].elapsed_time(m[i + 1]) for m in marks]))
        plan_ms, d_ms, c_ms = avg(0), avg(2), avg(4)
        half = (1 + w.k) * w.T * w.H * 2
        dc = 2 * half
        dname, cname = row_kernel_names(w.T, w.k, w.H)
        dom, dom_ms = (dname, d_ms) if d_ms >= c_ms else (cname, c_ms)
        gbps = dc / ((d_ms + c_ms) / 1e3) / 1e9
        out[w.name] = {
            "stage_us": {"plan": round(plan_ms * 1e3, 2), "dispatch": round(d_ms * 1e3, 2),
                         "combine": round(c_ms * 1e3, 2)},
            "dispatch_combine_GBps": round(gbps, 1), "frac_of_peak": round(gbps / PEAK_GBPS, 4),
            "routed_rows_per_s": round(w.T * w.k / ((d_ms + c_ms) / 1e3), 1),
            "roofline": {"bound": "hbm", "kernel": dom,
                         "achieved": round(half / (dom_ms / 1e3) / 1e9, 1), "peak": PEAK_GBPS,
                         "unit": "GB/s", "frac": round(half / (dom_ms / 1e3) / 1e9 / PEAK_GBPS, 4)}}
        del b
        torch.cuda.empty_cache()
    return out


def separate_calls_leg(P, b, flush, steps, ev, np, torch) -> dict:
    """Route, assignment and layout as three separate calls (the kernels of
    moe_route, moe_assign_replicas and moe_layout), each bracketed by events,
    for comparison with the one-call plan the headline step uses. A fill of
    the flush buffer first keeps the GPU busy while the host enqueues them,
    as in the headline step, so the brackets hold kernel time, not launch
    latency."""
    marks = []
    for i in range(steps + 2):
        if flush is not None:
            flush.fill_(8.0)
        e = [ev() for _ in range(4)]
        e[0].record()
        P.route(b)
        e[1].record()
        P.assign(b)
        e[2].record()
        P.layout(b)
        e[3].record()
        if i >= 2:
            marks.append(e)
    torch.cuda.synchronize()
    return {name: round(float(np.mean([m[i].elapsed_time(m[i + 1]) for m in marks])), 4)
            for i, name in enumerate(("route", "assign", "layout"))}


def path_summary(w, meta_ms: dict, disp_ms: float, comb_ms: float, dc_bytes: int) -> dict:
    """The whole forward path (the one-call route + assignment + layout, then
    dispatch and combine; the expert stand-in and the cache flushes excluded),
    kernel time summed per stage. Algorithmic bytes: dispatch and combine rows, the logits, and 32
    bytes of metadata per (token, slot) pair (route writes idx and w; layout
    reads idx and writes pos and src; dispatch reads pos; combine reads pos
    and w)."""
    ms = sum(meta_ms.values()) + disp_ms + comb_ms
    nbytes = dc_bytes + w.T * w.E * 4 + 32 * w.T * w.k
    return {"us": round(ms * 1e3, 2), "bytes": nbytes,
            "GBps": round(nbytes / (ms / 1e3) / 1e9, 2),
            "frac_of_peak": round(nbytes / (ms / 1e3) / 1e9 / PEAK_GBPS, 4),
            "routed_rows_per_s": round(w.T * w.k / (ms / 1e3), 1),
            "metadata_share_of_time": round(sum(meta_ms.values()) / ms, 4)}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              f"(the routing path is single-GPU; sharding is a design note only)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    from combine_router_topk_amd import binding as B
    from combine_router_topk_amd import path as P

    w = synth.BY_NAME[args.workload]
    # the oracle legs run first: the all-cores leg forks worker processes,
    # which must happen before this process touches the GPU
    cpu = None
    if args.cpu_tokens > 0:
        cpu = cpu_baseline(w, args.seed, args.cpu_tokens, args.cpu_seconds)
        cpu["all_cores"] = cpu_baseline_all_cores(w, args.seed, args.cpu_seconds)
        cpu["next_rows"] = cpu_next_rows(w, args.seed, args.cpu_tokens, args.cpu_seconds / 4)
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    logits = synth.make_logits(w, args.seed)
    x = synth.make_x(w, args.seed)
    rep = synth.replica_table(w)
    tdt = torch.float16 if w.act_dtype == synth.F16 else torch.bfloat16
    p = B.make_problem(w.T, w.E, w.k, w.H, w.R, w.act_dtype)
    b = P.allocate(p, torch.from_numpy(logits), torch.from_numpy(x.view(np.int16)).view(tdt),
                   None if rep is None else torch.from_numpy(rep), device=dev)
    flush = None if args.warm_cache else torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    ev = timing_event_type(B._lib, torch)
    marks, meta_marks = [], []

    def step(record: bool):
        m0, m1 = ev(), ev()
        m0.record()
        P.route_assign_layout(b)
        m1.record()
        if flush is not None:
            flush.fill_(1.0)
        e0, e1, e2, e3 = ev(), ev(), ev(), ev()
        e0.record()
        P.dispatch(b)
        e1.record()
        P.standin(b)
        if flush is not None:
            flush.fill_(2.0)
        e2.record()
        P.combine(b)
        e3.record()
        if record:
            marks.append((e0, e1, e2, e3))
            meta_marks.append((m0, m1))

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()

    meta_ms = {"plan": float(np.mean([a.elapsed_time(c) for a, c in meta_marks]))}
    disp_all = [a.elapsed_time(b_) for a, b_, _, _ in marks]
    comb_all = [c.elapsed_time(d) for _, _, c, d in marks]
    disp_ms, comb_ms = float(np.mean(disp_all)), float(np.mean(comb_all))
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    half = (1 + w.k) * w.T * w.H * 2            # bytes of each of dispatch and combine
    dc_bytes = 2 * half
    dc_s = (disp_ms + comb_ms) / 1e3
    value = dc_bytes / dc_s / 1e9
    dname, cname = row_kernel_names(w.T, w.k, w.H)
    dom, dom_ms = (dname, disp_ms) if disp_ms >= comb_ms else (cname, comb_ms)
    achieved = half / (dom_ms / 1e3) / 1e9
    traffic = traffic_from_profiles(dom, w.name)

    # a plain device copy of the dispatch's byte count (torch copy_, the
    # runtime's device-to-device copy), as an achievable-bandwidth reference
    cp_src = torch.empty(half // 4, dtype=torch.int16, device=dev)
    cp_dst = torch.empty_like(cp_src)
    cp_ms = []
    for i in range(6):
        if flush is not None:
            flush.fill_(3.0)
        a, c = ev(), ev()
        a.record()
        cp_dst.copy_(cp_src)
        c.record()
        if i > 0:
            cp_ms.append((a, c))
    torch.cuda.synchronize()
    copy_gbps = 2 * cp_src.numel() * 2 / (np.mean([a.elapsed_time(c) for a, c in cp_ms]) / 1e3) / 1e9
    # a write-only reference: torch's fill of the 1 GiB flush buffer
    fill_gbps = None
    if flush is not None:
        fl_ms = []
        for i in range(6):
            a, c = ev(), ev()
            a.record()
            flush.fill_(float(i))
            c.record()
            if i > 0:
                fl_ms.append((a, c))
        torch.cuda.synchronize()
        fill_gbps = FLUSH_BYTES / (np.mean([a.elapsed_time(c) for a, c in fl_ms]) / 1e3) / 1e9

    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype_name,
        "data": "synthetic",
        "config": {"workload": w.name, "T": w.T, "E": w.E, "k": w.k, "H": w.H, "R": w.R,
                   "act": w.dtype_name, "seed": args.seed,
                   "cache": "warm" if flush is None else "cold: 1 GiB fill before dispatch and before combine"},
        "frac_of_peak": round(value / PEAK_GBPS, 4),
        "routed_rows_per_s": round(w.T * w.k / dc_s, 1),
        "path": path_summary(w, meta_ms, disp_ms, comb_ms, dc_bytes),
        "stage_ms": {**{k_: round(v_, 4) for k_, v_ in meta_ms.items()},
                     "dispatch": round(disp_ms, 4), "combine": round(comb_ms, 4)},
        "separate_calls_ms": separate_calls_leg(P, b, flush, 20, ev, np, torch),
        "median_ms": {"dispatch": round(float(np.median(disp_all)), 4),
                      "combine": round(float(np.median(comb_all)), 4)},
        "dedup_rows": int(b.dedup.sum().item()),
        "raw_rows": w.T * w.k,
        "max_active_experts": int(b.active.max().item()),
        "copy_reference_GBps": round(copy_gbps, 1),
        "fill_reference_GBps": None if fill_gbps is None else round(fill_gbps, 1),
        "build_id": B.moe_build_id(),
        "inputs": {"numpy": np.__version__,
                   "logits_sha256": hashlib.sha256(logits.tobytes()).hexdigest()[:16],
                   "x_sha256": hashlib.sha256(x.tobytes()).hexdigest()[:16]},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 2),
                     "peak": PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / PEAK_GBPS, 4),
                     "traffic": traffic},
    }
    if args.workload_steps > 0:
        res["workloads"] = workloads_leg(P, B, synth, np, torch, dev, flush, ev, args.seed,
                                         args.workload_steps, w.name)
    if flush is not None and args.warm_steps > 0:
        res["warm_cache"] = warm_leg(P, b, args.warm_steps, ev, np, torch, dc_bytes)
    if args.single_send_steps > 0:
        res["single_send"] = single_send_leg(P, w, b, flush, args.single_send_steps, ev, np, torch)
    if args.backward_steps > 0:
        res["backward"] = backward_leg(B, w, b, flush, args.backward_steps, ev, np, torch, synth,
                                       args.seed)
    if args.stats_steps > 0:
        res["routing_stats"] = stats_leg(P, w, b, flush, args.stats_steps, ev, np, torch)
    if args.eplb_steps > 0:
        res["eplb"] = eplb_leg(P, B, synth, np, torch, dev, flush, args.eplb_steps, ev, args.seed)
    if args.graph_steps > 0:
        res["decode_graph"] = graph_leg(P, B, synth, np, torch, dev, args.graph_steps, args.seed)
    if cpu is not None:
        res["cpu_baseline"] = cpu
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
