"""Pins for the oracle's dispatch, expert stand-in and combine: byte equality,
16-bit rounding against torch's CPU conversions, exact closed forms, and the
k = 1 special case (no GPU)."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle.rows import BF16, F16


def test_encode16_matches_torch_rounding():
    rng = np.random.default_rng(0)
    f = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * 10,
        # exact halfway cases between neighbouring bf16 / fp16 values
        (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
        np.array([0.0, -0.0, 65504.0, 65520.0, 1e-8, -3.0e38], np.float32)])
    bf = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.encode16(f, BF16), bf)
    hf = torch.from_numpy(f).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.encode16(f, F16), hf)
    assert np.array_equal(oracle.decode16(bf, BF16),
                          torch.from_numpy(bf.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_dispatch_is_bit_copy_including_nan_patterns():
    rng = np.random.default_rng(1)
    T, k, H = 37, 3, 24
    x = rng.integers(0, 65536, size=(T, H), dtype=np.uint16)    # any bit pattern
    pos = rng.permutation(T * k).astype(np.int32)
    send = oracle.dispatch(x, pos, k)
    for i in range(T * k):
        assert send[pos[i]].tobytes() == x[i // k].tobytes()
    src = np.empty_like(pos)
    src[pos] = np.arange(T * k)
    rows = np.array([0, 5, T * k - 1])
    assert np.array_equal(oracle.dispatch_rows(x, src, k, rows), send[rows])


@pytest.mark.parametrize("act", [F16, BF16])
@pytest.mark.parametrize("E", [8, 64, 256])
def test_standin_is_single_rounding_of_exact_product(act, E):
    rng = np.random.default_rng(E + act)
    n, H = 64, 32
    f = rng.standard_normal((n, H)).astype(np.float32)
    bits = oracle.encode16(f, act)
    e = rng.integers(0, E, n)
    y = oracle.expert_standin(bits, e, E, act)
    exact = oracle.decode16(bits, act).astype(np.float64) * (1.0 + e / E)[:, None]  # exact in fp64
    tdt = torch.float16 if act == F16 else torch.bfloat16
    ref = torch.from_numpy(exact).to(tdt).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(y, ref)


def test_combine_exact_closed_form():
    # x values with few significant bits keep y = x*(1+e/E) exact, so
    # out[t] = x[t] * sum_j w_j (1 + e_j/E) holds to fp64 rounding
    rng = np.random.default_rng(2)
    T, E, k, H, R = 40, 8, 3, 16, 4
    l = rng.standard_normal((T, E)).astype(np.float32)
    xs = rng.choice([-2.0, -1.5, -1.0, -0.5, 0.0, 0.5, 1.0, 1.5, 2.0], size=(T, H)).astype(np.float32)
    for act in (F16, BF16):
        x = oracle.encode16(xs, act)
        m = oracle.route_and_layout(T, E, k, R, l)
        r = oracle.rows_for(m, x, E, k, act)
        for t in range(T):
            s = sum(float(m["w"][t, j]) * (1.0 + int(m["idx"][t, j]) / E) for j in range(k))
            ref = xs[t].astype(np.float64) * s
            assert np.allclose(r["out"][t], ref, rtol=1e-12, atol=1e-15)


def test_combine_top1_returns_stand_in_row():
    rng = np.random.default_rng(3)
    T, E, H = 30, 8, 16
    l = rng.standard_normal((T, E)).astype(np.float32)
    x = oracle.encode16(rng.standard_normal((T, H)).astype(np.float32), BF16)
    m = oracle.route_and_layout(T, E, 1, 2, l)
    r = oracle.rows_for(m, x, E, 1, BF16)
    y_tok = r["y"][m["pos"]]      # y row of each token
    assert np.array_equal(r["out"], oracle.decode16(y_tok, BF16).astype(np.float64))


def test_rows_for_subset_matches_full():
    w = synth.scaled(synth.TRAIN_TOP6, T=300, H=64)
    l = synth.make_logits(w, 1)
    x = synth.make_x(w, 1)
    m = oracle.route_and_layout(w.T, w.E, w.k, w.R, l)
    full = oracle.rows_for(m, x, w.E, w.k, w.act_dtype)
    rows = np.array([0, 17, w.T * w.k - 1])
    toks = np.array([5, 299, 0])
    sub = oracle.rows_for(m, x, w.E, w.k, w.act_dtype, send_rows=rows, tokens=toks)
    assert np.array_equal(sub["send"], full["send"][rows])
    assert np.array_equal(sub["y"], full["y"][rows])
    assert np.array_equal(sub["out"], full["out"][toks])
    # the closed form within the 16-bit rounding of y: |y - x(1+e/E)| <= 2^-8 |x(1+e/E)|
    xs = oracle.decode16(x, w.act_dtype).astype(np.float64)
    for t in (0, 100, 299):
        s = sum(float(m["w"][t, j]) * (1 + int(m["idx"][t, j]) / w.E) for j in range(w.k))
        bound = 2.0 ** -8 * np.abs(xs[t]) * s + 1e-30
        assert (np.abs(full["out"][t] - xs[t] * s) <= bound).all()
    assert not math.isnan(full["out"].sum())
