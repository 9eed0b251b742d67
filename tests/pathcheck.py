"""Helpers for the GPU parity tests: run the HIP path through the C ABI on
seeded inputs and compare every output with the CPU oracle.

Bars: bit-exact for every index, count, offset and row output; gate weights
within rtol 1e-6; the combine within |out - ref| <= 1e-3 + 4e-3 |ref| for the
16-bit output (ref = the oracle's fp64 sum) and within the fp32 accumulation
bound k * 2^-24 * sum_j |w_j y_j| for the fp32 output.
"""
from __future__ import annotations

import os
import sys

import numpy as np
import torch

import oracle
import synth
from combine_router_topk_amd import binding as B
from combine_router_topk_amd import path as P

W_RTOL = 1e-6
OUT_RTOL, OUT_ATOL = 4e-3, 1e-3


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def torch_act(act: int):
    return torch.float16 if act == synth.F16 else torch.bfloat16


def bits_to_tensor(bits: np.ndarray, act: int) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch_act(act))


def tensor_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def run_gpu(w: synth.Workload, logits: np.ndarray, x: np.ndarray, rep: np.ndarray | None,
            flags: int = 0, inplace_standin: bool = False) -> P.Buffers:
    p = B.make_problem(w.T, w.E, w.k, w.H, w.R, w.act_dtype, flags)
    b = P.allocate(p, torch.from_numpy(logits), bits_to_tensor(x, w.act_dtype),
                   None if rep is None else torch.from_numpy(rep))
    if inplace_standin:
        b.y = b.send
    P.run(b)
    torch.cuda.synchronize()
    return b


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


META_KEYS = ("counts", "assign", "active", "rank_of", "expert_offsets", "rank_offsets", "pos",
             "src", "dedup")


def check_meta(b: P.Buffers, ref: dict, T: int, k: int) -> None:
    assert np.array_equal(host(b.idx).reshape(T, k), ref["idx"]), "idx"
    for key in META_KEYS:
        got = host(getattr(b, key))
        assert np.array_equal(got, ref[key]), (key, got[:16], ref[key][:16])
    wg = host(b.w).reshape(T, k).astype(np.float64)
    wr = ref["w"].astype(np.float64)
    assert np.array_equal(np.isnan(wg), np.isnan(wr)), "w NaN pattern"
    bad = np.abs(wg - wr) > W_RTOL * np.abs(wr)
    assert not bad.any(), ("w", np.argwhere(bad)[:5], wg[bad][:5], wr[bad][:5])


def check_rows(b: P.Buffers, ref: dict, x: np.ndarray, w: synth.Workload,
               send_rows: np.ndarray | None, tokens: np.ndarray | None, out_f32: bool,
               check_send: bool = True) -> None:
    r = oracle.rows_for(ref, x, w.E, w.k, w.act_dtype, send_rows=send_rows, tokens=tokens)
    rows_t = torch.from_numpy(r["send_rows"]).to(b.send.device, torch.int64)
    if check_send:
        got_send = tensor_bits(b.send.index_select(0, rows_t))
        assert np.array_equal(got_send, r["send"]), "send rows"
    got_y = tensor_bits(b.y.index_select(0, rows_t))
    if not np.array_equal(got_y, r["y"]):
        bad = np.argwhere(got_y != r["y"])[:8]
        flat = ref["idx"].ravel()
        detail = [(int(r["send_rows"][i]), int(c), hex(int(r["send"][i, c])),
                   int(flat[ref["src"][r["send_rows"][i]]]), hex(int(got_y[i, c])), hex(int(r["y"][i, c])))
                  for i, c in bad]
        raise AssertionError(f"y rows: {int((got_y != r['y']).sum())} mismatches; "
                             f"(row, col, send bits, expert, got, want): {detail}")
    tok_t = torch.from_numpy(r["tokens"]).to(b.out.device, torch.int64)
    got = b.out.index_select(0, tok_t).float().cpu().numpy().astype(np.float64)
    refo = r["out"]
    if out_f32:
        # fp32 accumulation bound: k roundings of at most 2^-24 of the running sum
        mag = np.zeros_like(refo)
        toks = r["tokens"]
        for j in range(w.k):
            rows = ref["pos"][toks * w.k + j]
            yrow = oracle.decode16(oracle.expert_standin(
                oracle.dispatch_rows(x, ref["src"], w.k, rows), ref["idx"].ravel()[ref["src"][rows]],
                w.E, w.act_dtype), w.act_dtype).astype(np.float64)
            mag += np.abs(ref["w"][toks, j].astype(np.float64))[:, None] * np.abs(yrow)
        bound = w.k * 2.0 ** -24 * mag + 1e-30
        bad = np.abs(got - refo) > bound
    else:
        bad = np.abs(got - refo) > OUT_ATOL + OUT_RTOL * np.abs(refo)
    assert not bad.any(), ("out", np.argwhere(bad)[:5], got[bad][:5], refo[bad][:5])


# ---- full-size comparisons, every element ------------------------------------

def token_chunks(T: int, k: int, H: int, max_elems: int = 1 << 26, min_chunks: int = 16):
    """Token ranges [t0, t1) covering the batch, each small enough that one
    chunk's rows (about k*H elements per token) stay a few hundred MB on the
    host, and at least min_chunks of them so the thread pool has work."""
    per = max(1, min(max_elems // max(1, k * H), -(-T // min_chunks)))
    return [(t0, min(T, t0 + per)) for t0 in range(0, T, per)]


def run_chunked(gather, check, chunks, workers: int = 16) -> None:
    """gather(t0, t1) runs on the calling thread (device-to-host copies in
    stream order) and returns host arrays; check(t0, t1, *arrays) runs the
    oracle and the comparison on a thread pool (numpy releases the GIL in its
    array loops). At most 2 * workers chunks are in flight; the first failure
    is raised."""
    from concurrent.futures import ThreadPoolExecutor
    workers = max(1, min(workers, os.cpu_count() or 1))
    pending = []
    with ThreadPoolExecutor(max_workers=workers) as ex:
        for t0, t1 in chunks:
            arrays = gather(t0, t1)
            pending.append(ex.submit(check, t0, t1, *arrays))
            if len(pending) >= 2 * workers:
                pending.pop(0).result()
        for f in pending:
            f.result()


def chunk_rows(ref: dict, k: int, t0: int, t1: int):
    """The send rows of tokens [t0, t1) in (token, slot) order, and a pos table
    into a compact array holding them in that order."""
    items = np.arange(t0 * k, t1 * k)
    rows = ref["pos"][items].astype(np.int64)
    pos_c = np.zeros(ref["pos"].shape[0], dtype=np.int64)
    pos_c[items] = np.arange(items.shape[0])
    return rows, pos_c


def oracle_y(ref: dict, x: np.ndarray, w: synth.Workload, rows: np.ndarray) -> np.ndarray:
    """The oracle's stand-in rows for the given send rows, from their own
    dispatch rows."""
    flat = ref["idx"].ravel()
    return oracle.expert_standin(oracle.dispatch_rows(x, ref["src"], w.k, rows),
                                 flat[ref["src"][rows]], w.E, w.act_dtype)


def check_rows_all(b: P.Buffers, ref: dict, x: np.ndarray, w: synth.Workload) -> None:
    """Every stand-in row bit for bit and every combine output element within
    1e-3 + 4e-3 |ref| against the oracle, token chunk by token chunk (each
    chunk's k T_c send rows and T_c output rows)."""
    k = w.k

    def gather(t0, t1):
        rows, _ = chunk_rows(ref, k, t0, t1)
        rt = torch.from_numpy(rows).to(b.y.device)
        return (tensor_bits(b.y.index_select(0, rt)),
                b.out[t0:t1].float().cpu().numpy())

    def check(t0, t1, got_y, got_out):
        rows, pos_c = chunk_rows(ref, k, t0, t1)
        y_ref = oracle_y(ref, x, w, rows)
        if not np.array_equal(got_y, y_ref):
            bad = np.argwhere(got_y != y_ref)[:6]
            raise AssertionError(f"y rows of tokens [{t0}, {t1}): {int((got_y != y_ref).sum())} "
                                 f"mismatches at (send row, col) {[(int(rows[i]), int(c)) for i, c in bad]}")
        out_ref = oracle.combine(y_ref, pos_c, ref["w"], k, w.act_dtype, np.arange(t0, t1))
        got = got_out.astype(np.float64)
        bad = np.abs(got - out_ref) > OUT_ATOL + OUT_RTOL * np.abs(out_ref)
        assert not bad.any(), ("out", t0, np.argwhere(bad)[:5], got[bad][:5], out_ref[bad][:5])

    run_chunked(gather, check, token_chunks(w.T, k, w.H))
