"""GPU parity of the backward of the combine (dy, dw) and of the dispatch (dx)
against the CPU oracle, through the C ABI, on the layout the GPU forward
wrote (itself checked against the oracle first).

Bars: dy bit-exact (one fp32 product rounded once to the activation
format on both sides); dw within the fp32 summation bound
H * 2^-24 * sum_h |y_h dout_h| of the oracle's exact value (every product of
two 16-bit values is exact in fp32); dx within 1e-3 + 4e-3 |ref| in the
activation format and within k * 2^-24 * sum_j |dsend_j| with fp32 output.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from combine_router_topk_amd import binding as B
from pathcheck import (bits_to_tensor, check_meta, chunk_rows, host, oracle_y, run_chunked, run_gpu,
                       say, tensor_bits, token_chunks)

pytestmark = pytest.mark.gpu

U24 = 2.0 ** -24
OUT_RTOL, OUT_ATOL = 4e-3, 1e-3


def dec(bits, act):
    return oracle.decode16(bits, act).astype(np.float64)


def oracle_rows(ref, x, w, rows):
    """The oracle's y rows (stand-in of the dispatched rows) for send rows."""
    flat = ref["idx"].ravel()
    return oracle.expert_standin(oracle.dispatch_rows(x, ref["src"], w.k, rows),
                                 flat[ref["src"][rows]], w.E, w.act_dtype)


def compact(ref, k, tokens):
    """Send rows read by the chosen tokens and a pos table into them."""
    items = (tokens[:, None] * k + np.arange(k)[None, :]).ravel()
    need = ref["pos"][items]
    pos_c = np.zeros(ref["pos"].shape[0], dtype=np.int64)
    pos_c[items] = np.arange(items.shape[0])
    return need, pos_c


def check_dw(got_dw, ref, x, w, dout, tokens):
    need, pos_c = compact(ref, w.k, tokens)
    y_need = oracle_rows(ref, x, w, need)
    want = oracle.combine_backward_dw(y_need, dout, pos_c, w.k, w.act_dtype, tokens)
    g = dec(dout[tokens], w.act_dtype)
    mag = np.stack([(np.abs(dec(y_need[pos_c[tokens * w.k + j]], w.act_dtype)) * np.abs(g)).sum(1)
                    for j in range(w.k)], axis=1)
    bound = w.H * U24 * mag + 1e-30
    got = got_dw.reshape(w.T, w.k)[tokens].astype(np.float64)
    bad = np.abs(got - want) > bound
    assert not bad.any(), ("dw", np.argwhere(bad)[:5], got[bad][:5], want[bad][:5])


def check_dx(got_dx, dsend_rows_fn, ref, w, tokens, out_f32):
    need, pos_c = compact(ref, w.k, tokens)
    ds = dsend_rows_fn(need)
    want = oracle.dispatch_backward(ds, pos_c, w.k, w.act_dtype, tokens, T=w.T)
    got = got_dx[tokens].astype(np.float64)
    if out_f32:
        mag = sum(np.abs(dec(ds[pos_c[tokens * w.k + j]], w.act_dtype)) for j in range(w.k))
        bad = np.abs(got - want) > w.k * U24 * mag + 1e-30
    else:
        bad = np.abs(got - want) > OUT_ATOL + OUT_RTOL * np.abs(want)
    assert not bad.any(), ("dx", np.argwhere(bad)[:5], got[bad][:5], want[bad][:5])


def run_backward(w, seed, flags=0, dsend="grad", alias=False, outputs=("dy", "dw"),
                 dy_rows=None, tokens=None):
    say(f"[case] backward {w.name} seed={seed} flags={flags} dsend={dsend} alias={alias} "
        f"outputs={outputs}")
    logits, x = synth.make_logits(w, seed), synth.make_x(w, seed)
    rep = synth.replica_table(w)
    ref = oracle.route_and_layout(w.T, w.E, w.k, w.R, logits, rep)
    b = run_gpu(w, logits, x, rep)
    check_meta(b, ref, w.T, w.k)
    dout = synth.make_grad(w, seed, w.T)
    p = B.make_problem(w.T, w.E, w.k, w.H, w.R, w.act_dtype, flags)
    g = bits_to_tensor(dout, w.act_dtype).cuda()
    n = w.T * w.k
    dy = (b.y if alias else torch.empty_like(b.y)) if "dy" in outputs else None
    dw = torch.empty(n, dtype=torch.float32, device="cuda") if "dw" in outputs else None
    B.moe_combine_backward(p, g, b.y if "dw" in outputs else None, b.pos,
                           b.w if "dy" in outputs else None, dy, dw)
    torch.cuda.synchronize()
    rows = np.arange(n) if dy_rows is None else dy_rows
    toks = np.arange(w.T) if tokens is None else tokens
    # dy is formed from the gate weights the kernel was given (the GPU's, equal
    # to the oracle's within rtol 1e-6, checked above), so the bit-exact
    # comparison does not hang on a last-place difference in w
    w_gpu = host(b.w).reshape(w.T, w.k)
    if dy is not None:
        want = oracle.combine_backward_dy(dout, ref["src"], w_gpu, w.k, w.act_dtype, rows)
        got = tensor_bits(dy.index_select(0, torch.from_numpy(rows).cuda()))
        if not np.array_equal(got, want):
            bad = np.argwhere(got != want)[:6]
            raise AssertionError(f"dy: {int((got != want).sum())} mismatches at (row, col) "
                                 f"{[(int(rows[i]), int(c)) for i, c in bad]}: got "
                                 f"{[hex(int(got[i, c])) for i, c in bad]} want "
                                 f"{[hex(int(want[i, c])) for i, c in bad]}")
    if dw is not None:
        check_dw(host(dw), ref, x, w, dout, toks)
    # dispatch backward: independent gradient rows, or the dy just computed
    out_f32 = bool(flags & B.MOE_FLAG_OUT_F32)
    if dsend == "grad":
        ds_bits = synth.make_grad(w, seed, n, stream=1)
        ds = bits_to_tensor(ds_bits, w.act_dtype).cuda()
        rows_fn = lambda r: ds_bits[r]
    else:
        ds = dy
        rows_fn = lambda r: oracle.combine_backward_dy(dout, ref["src"], w_gpu, w.k, w.act_dtype, r)
    dx = torch.empty(w.T, w.H, dtype=torch.float32 if out_f32 else b.x.dtype, device="cuda")
    B.moe_dispatch_backward(p, ds, b.pos, dx)
    torch.cuda.synchronize()
    check_dx(dx.float().cpu().numpy(), rows_fn, ref, w, toks, out_f32)
    return b, g, dx


SMALL = [
    synth.TINY,
    synth.DECODE,
    synth.scaled(synth.TRAIN_TOP2, T=3001, H=512),
    synth.scaled(synth.TRAIN_TOP6, T=2053, H=264),
    synth.scaled(synth.LARGE, T=777, H=7168),
]


@pytest.mark.parametrize("seed", [0, 1])
@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_backward_small(w, seed):
    run_backward(w, seed)


@pytest.mark.parametrize("w", [synth.TINY, synth.scaled(synth.TRAIN_TOP6, T=999, H=128),
                               synth.scaled(synth.LARGE, T=300, H=1024)], ids=lambda w: w.name)
def test_backward_fp32_dx(w):
    run_backward(w, 1, flags=B.MOE_FLAG_OUT_F32)


# The second workload of each pair is split into a dw launch and a sliced dy
# launch (rows over 256 chunks, k >= 5, k dy rows of at least 64 KiB, at
# least 8192 slices): dy alone then runs only the slices, and dy in place of
# y needs dw's reads of y to come first.
SPLIT = synth.scaled(synth.LARGE, T=1200, H=7168)


@pytest.mark.parametrize("outputs", [("dy",), ("dw",)])
@pytest.mark.parametrize("w", [synth.scaled(synth.TRAIN_TOP6, T=700, H=520), SPLIT], ids=lambda w: w.name)
def test_backward_single_output(w, outputs):
    run_backward(w, 2, outputs=outputs)


@pytest.mark.parametrize("w", [synth.scaled(synth.TRAIN_TOP2, T=1000, H=256), SPLIT], ids=lambda w: w.name)
def test_backward_dy_in_place_of_y(w):
    run_backward(w, 3, alias=True)


def test_backward_chain_dsend_is_dy():
    run_backward(synth.scaled(synth.TRAIN_TOP6, T=1500, H=128), 4, dsend="dy")


EDGE = [
    ("E1_k1_R1_H8", 1, 1, 1, 1, 8),         # one chunk per row, 16-lane teams
    ("E5_k3_R5_H24", 97, 5, 3, 5, 24),
    ("E8_k8_H16", 300, 8, 8, 2, 16),        # k = E
    ("E12_k5_R3_H40", 513, 12, 5, 3, 40),
    ("E100_k7_R10_H504", 611, 100, 7, 10, 504),   # 63 chunks: the widest team inside a wave
    ("E384_k10_R12_H64", 700, 384, 10, 12, 64),
    ("E1024_k16_R1024_H16", 300, 1024, 16, 1024, 16),
    ("T1", 1, 64, 2, 32, 4096),
]


@pytest.mark.parametrize("name,T,E,k,R,H", EDGE, ids=[e[0] for e in EDGE])
def test_backward_edge_shapes(name, T, E, k, R, H):
    run_backward(synth.Workload(name, T, E, k, H, R, synth.BF16, "none", False), 5)


# Row widths (16-byte chunks per row: 129 and 256, the one-row blocks with
# one chunk position per step and the pos entries loaded by lanes; then 257,
# 375, 513, 1024, 1537, two chunk positions per step), k up to 8.
WIDTHS = [("H1032_k5", 1032, 5), ("H2048_k2", 2048, 2), ("H2056_k3", 2056, 3),
          ("H3000_k8", 3000, 8), ("H4104_k4", 4104, 4), ("H8192_k6", 8192, 6),
          ("H12296_k7", 12296, 7)]


@pytest.mark.parametrize("name,H,k", WIDTHS, ids=[v[0] for v in WIDTHS])
def test_backward_row_widths(name, H, k):
    run_backward(synth.Workload(name, 300, 16, k, H, 4, synth.BF16, "zipf1.2", False), 6)


# The dispatch backward in row slices (rows over 256 chunks, launches of at
# least 12288 slices), at each of its LDS reservations (k = 2, 3, 4..6, 8)
# and with ragged last slices (257, 375, 513 and 1537 chunks); at 1537
# chunks with k = 6 the combine backward is split into dw and sliced dy.
SLICED = [("H2056_k3_T4200", 2056, 3, 4200), ("H3000_k8_T4200", 3000, 8, 4200),
          ("H4104_k4_T2500", 4104, 4, 2500), ("H12296_k2_T1000", 12296, 2, 1000),
          ("H12296_k6_T1000", 12296, 6, 1000)]


@pytest.mark.parametrize("name,H,k,T", SLICED, ids=[v[0] for v in SLICED])
def test_backward_sliced_row_widths(name, H, k, T):
    run_backward(synth.Workload(name, T, 16, k, H, 4, synth.BF16, "zipf1.2", False), 7)


def test_backward_empty_batch_and_errors():
    w = synth.Workload("bwd_empty", 0, 8, 2, 128, 4, synth.F16, "none", False)
    say("[case] backward empty batch and argument errors")
    p = B.make_problem(w.T, w.E, w.k, w.H, w.R, w.act_dtype)
    e = torch.empty(0, dtype=torch.float16, device="cuda")
    i = torch.empty(0, dtype=torch.int32, device="cuda")
    f = torch.empty(0, dtype=torch.float32, device="cuda")
    B.moe_combine_backward(p, e, e, i, f, e, f)
    B.moe_dispatch_backward(p, e, i, e)
    p1 = B.make_problem(4, w.E, w.k, w.H, w.R, w.act_dtype)
    g = torch.zeros(4, w.H, dtype=torch.float16, device="cuda")
    pos = torch.arange(8, dtype=torch.int32, device="cuda")
    with pytest.raises(B.MoeError) as ei:
        B.moe_combine_backward(p1, g, None, pos, None, None, None)
    assert ei.value.status == B.MOE_ERR_INVALID_ARG


# every workload at seeds 0 and 1
FULL_CASES = [(w, s) for w in (synth.DECODE, synth.TRAIN_TOP2, synth.TRAIN_TOP6, synth.LARGE) for s in (0, 1)]


@pytest.mark.parametrize("w,seed", FULL_CASES, ids=lambda v: v.name if hasattr(v, "name") else f"seed{v}")
def test_backward_full_size(w, seed):
    """Full size, every element, token chunk by token chunk: dy bit for bit,
    dw within its fp32 summation bound and dx (from dsend = dy) within
    1e-3 + 4e-3 |ref| against the oracle; and dx against the property
    sum_j w_j = 1 (dx = dout up to the roundings of dy, the fp32 sum and dx)."""
    say(f"[case] backward full {w.name} seed {seed}")
    logits, x = synth.make_logits(w, seed), synth.make_x(w, seed)
    rep = synth.replica_table(w)
    ref = oracle.route_and_layout(w.T, w.E, w.k, w.R, logits, rep)
    b = run_gpu(w, logits, x, rep)
    check_meta(b, ref, w.T, w.k)
    dout = synth.make_grad(w, seed, w.T)
    p = B.make_problem(w.T, w.E, w.k, w.H, w.R, w.act_dtype)
    g = bits_to_tensor(dout, w.act_dtype).cuda()
    dy = torch.empty_like(b.y)
    dw = torch.empty(w.T * w.k, dtype=torch.float32, device="cuda")
    dx = torch.empty_like(b.x)
    B.moe_combine_backward(p, g, b.y, b.pos, b.w, dy, dw)
    B.moe_dispatch_backward(p, dy, b.pos, dx)
    torch.cuda.synchronize()
    w_gpu = host(b.w).reshape(w.T, w.k)
    k = w.k

    def gather(t0, t1):
        rows, _ = chunk_rows(ref, k, t0, t1)
        rt = torch.from_numpy(rows).cuda()
        return (tensor_bits(dy.index_select(0, rt)), host(dw[t0 * k:t1 * k]).reshape(t1 - t0, k),
                dx[t0:t1].float().cpu().numpy())

    def check(t0, t1, got_dy, got_dw, got_dx):
        rows, pos_c = chunk_rows(ref, k, t0, t1)
        toks = np.arange(t0, t1)
        dy_ref = oracle.combine_backward_dy(dout, ref["src"], w_gpu, k, w.act_dtype, rows)
        if not np.array_equal(got_dy, dy_ref):
            bad = np.argwhere(got_dy != dy_ref)[:6]
            raise AssertionError(f"dy of tokens [{t0}, {t1}): {int((got_dy != dy_ref).sum())} "
                                 f"mismatches at (send row, col) {[(int(rows[i]), int(c)) for i, c in bad]}")
        y_ref = oracle_y(ref, x, w, rows)
        dw_ref = oracle.combine_backward_dw(y_ref, dout, pos_c, k, w.act_dtype, toks)
        gd = dec(dout[toks], w.act_dtype)
        mag = np.stack([(np.abs(dec(y_ref[pos_c[toks * k + j]], w.act_dtype)) * np.abs(gd)).sum(1)
                        for j in range(k)], axis=1)
        bad = np.abs(got_dw.astype(np.float64) - dw_ref) > w.H * U24 * mag + 1e-30
        assert not bad.any(), ("dw", t0, np.argwhere(bad)[:5])
        dx_ref = oracle.dispatch_backward(dy_ref, pos_c, k, w.act_dtype, toks, T=w.T)
        bad = np.abs(got_dx.astype(np.float64) - dx_ref) > OUT_ATOL + OUT_RTOL * np.abs(dx_ref)
        assert not bad.any(), ("dx", t0, np.argwhere(bad)[:5])

    run_chunked(gather, check, token_chunks(w.T, k, w.H))
    u16 = 2.0 ** -11 if w.act_dtype == synth.F16 else 2.0 ** -8
    rel = 2 * u16 + (2 * w.k + 2) * U24
    step = 1 << 12
    for t0 in range(0, w.T, step):
        gg = g[t0:t0 + step].float()
        err = (dx[t0:t0 + step].float() - gg).abs()
        assert bool((err <= rel * gg.abs() + 2.0 ** -23).all()), t0


def test_backward_deterministic_bitwise():
    """dw and dx are fp32 sums in a fixed order: two runs give the same bits."""
    w = synth.scaled(synth.TRAIN_TOP6, T=3000, H=520)
    say("[case] backward determinism")
    logits, x = synth.make_logits(w, 9), synth.make_x(w, 9)
    b = run_gpu(w, logits, x, None)
    p = B.make_problem(w.T, w.E, w.k, w.H, w.R, w.act_dtype, B.MOE_FLAG_OUT_F32)
    g = bits_to_tensor(synth.make_grad(w, 9, w.T), w.act_dtype).cuda()
    outs = []
    for _ in range(2):
        dy = torch.empty_like(b.y)
        dw = torch.empty(w.T * w.k, dtype=torch.float32, device="cuda")
        dx = torch.empty(w.T, w.H, dtype=torch.float32, device="cuda")
        B.moe_combine_backward(p, g, b.y, b.pos, b.w, dy, dw)
        B.moe_dispatch_backward(p, dy, b.pos, dx)
        torch.cuda.synchronize()
        outs.append((dy.view(torch.int16).clone(), dw.view(torch.int32).clone(),
                     dx.view(torch.int32).clone()))
    for a, c in zip(*outs):
        assert torch.equal(a, c)
