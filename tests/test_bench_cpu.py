"""The benchmark's host-side parts without a GPU: it refuses more than one
GPU before touching the device, and its oracle baselines (dispatch+combine,
and the rows beyond it) run on a small sample and report the fields the
JSON line carries."""
import os
import subprocess
import sys

import synth
from conftest import ROOT

sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_cpu_baseline_fields():
    w = synth.scaled(synth.TRAIN_TOP2, T=64, H=64)
    c = bench.cpu_baseline(w, 0, 64, 0.0)
    assert set(c) >= {"value", "unit", "cores", "kind", "sample"}
    assert c["unit"] == "GB/s" and c["kind"] == "oracle" and c["cores"] == 1 and c["value"] > 0


def test_cpu_next_rows_fields():
    w = synth.scaled(synth.TRAIN_TOP2, T=64, H=64)
    n = bench.cpu_next_rows(w, 0, 64, 0.0)
    assert n["single_send"]["dispatch_GBps"] > 0 and n["single_send"]["expand_GBps"] > 0
    assert n["backward"]["combine_backward_GBps"] > 0 and n["backward"]["dispatch_backward_GBps"] > 0
    assert n["routing_stats_pairs_per_s"] > 0 and n["token_balanced_split_pairs_per_s"] > 0


def test_timing_events_resolve_through_the_library():
    """The bench's timing events come from the HIP runtime the routing
    library is linked against (no event is created without a GPU)."""
    import torch
    from combine_router_topk_amd import binding as B
    Ev = bench.timing_event_type(B._lib, torch)
    assert callable(Ev) and {"record", "elapsed_time"} <= set(dir(Ev))


def test_path_summary_arithmetic():
    # train top-2: 768 MiB of rows + 4 MiB of logits + 32 B per pair, over
    # 100 us of summed stage time
    w = synth.TRAIN_TOP2
    dc = w.dispatch_combine_bytes()
    s = bench.path_summary(w, {"route": 0.005, "assign": 0.005, "layout": 0.01}, 0.04, 0.04, dc)
    want = 805_306_368 + 16384 * 64 * 4 + 32 * 16384 * 2
    assert s["bytes"] == want and s["us"] == 100.0
    assert abs(s["GBps"] - want / 100e-6 / 1e9) < 0.01
    assert s["metadata_share_of_time"] == 0.2
    assert abs(s["routed_rows_per_s"] - 32768 / 100e-6) < 1


def test_cpu_all_cores_fields():
    w = synth.scaled(synth.TRAIN_TOP2, T=96, H=64)
    c = bench.cpu_baseline_all_cores(w, 0, 0.0)
    assert c["unit"] == "GB/s" and c["kind"] == "oracle" and c["value"] > 0
    assert 1 <= c["cores"] <= 16 and c["cores"] == bench.host_cores()
    assert c["routed_rows_per_s"] > 0


def test_oracle_chunk_worker_keeps_the_full_layout_order():
    """A worker's chunk is dispatched in the order its pairs have in the
    whole send buffer: its rows are the whole batch's rows of those tokens."""
    import numpy as np
    import oracle
    w = synth.scaled(synth.TRAIN_TOP6, T=40, H=16)
    logits, x = synth.make_logits(w, 0), synth.make_x(w, 0)
    m = oracle.route_and_layout(w.T, w.E, w.k, w.R, logits)
    full = oracle.dispatch(x, m["pos"], w.k)
    t0, t1 = 7, 23
    loc, row_e = bench.chunk_layout(m["pos"], m["idx"], w.k, t0, t1)
    part = oracle.dispatch(x[t0:t1], loc, w.k)
    rows = np.sort(m["pos"][t0 * w.k:t1 * w.k])
    assert np.array_equal(part, full[rows])
    assert np.array_equal(row_e, m["idx"].ravel()[m["src"][rows]])
