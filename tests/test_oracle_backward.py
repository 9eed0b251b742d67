"""Pins for the oracle's backward of the dispatch and the combine: a
hand-worked example, the adjoint identities that define a gradient of a
linear map (checked against the forward oracle), the derivative of the loss
in the gate weights, and the k = 1 special case (no GPU)."""
import numpy as np
import pytest

import oracle
import synth
from conftest import load_golden

F16, BF16 = synth.F16, synth.BF16


def enc(a, act):
    return oracle.encode16(np.asarray(a, np.float32), act)


@pytest.mark.parametrize("act", [F16, BF16])
def test_handworked(act):
    g = load_golden("backward_handworked.json")
    k = g["k"]
    idx = np.array(g["idx"], np.int32)
    pos, src = oracle.permutation(idx, np.array(g["rank_of"], np.int32))
    assert pos.tolist() == g["pos"] and src.tolist() == g["src"]
    w = np.array(g["w"], np.float32)
    dout, y, dsend = enc(g["dout"], act), enc(g["y"], act), enc(g["dsend"], act)
    dy = oracle.combine_backward_dy(dout, src, w, k, act)
    assert np.array_equal(dy, enc(g["dy"], act))           # bits, so the -0 counts
    assert np.signbit(oracle.decode16(dy, act)[4, 0])
    assert np.array_equal(oracle.combine_backward_dw(y, dout, pos, k, act), np.array(g["dw"]))
    assert np.array_equal(oracle.dispatch_backward(dsend, pos, k, act), np.array(g["dx"]))
    # a subset of rows / tokens gives the same entries
    assert np.array_equal(oracle.combine_backward_dy(dout, src, w, k, act, rows=np.array([5, 1])),
                          enc(g["dy"], act)[[5, 1]])
    assert np.array_equal(oracle.combine_backward_dw(y, dout, pos, k, act, tokens=np.array([2])),
                          np.array(g["dw"])[[2]])
    assert np.array_equal(oracle.dispatch_backward(dsend, pos, k, act, tokens=np.array([1])),
                          np.array(g["dx"])[[1]])


def layout(T, E, k, R, seed):
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    return oracle.route_and_layout(T, E, k, R, logits)


def small_ints(rng, shape, act):
    return enc(rng.integers(-8, 9, size=shape), act)


@pytest.mark.parametrize("act", [F16, BF16])
@pytest.mark.parametrize("T,E,k,R", [(64, 8, 2, 4), (200, 16, 4, 4), (97, 12, 5, 3)])
def test_combine_adjoint_exact(T, E, k, R, act):
    """<combine(y, w), dout> = <y, dy> for every y: dy is the adjoint of the
    combine in y. Small integers and gate weights in quarters keep every
    product and rounding exact, so the identity holds exactly."""
    m = layout(T, E, k, R, T)
    rng = np.random.default_rng(1 + T)
    H = 16
    w = (rng.integers(0, 5, size=(T, k)) / 4).astype(np.float32)
    y, dout = small_ints(rng, (T * k, H), act), small_ints(rng, (T, H), act)
    out = oracle.combine(y, m["pos"], w, k, act)
    lhs = (out * oracle.decode16(dout, act).astype(np.float64)).sum()
    dy = oracle.combine_backward_dy(dout, m["src"], w, k, act)
    rhs = (oracle.decode16(y, act).astype(np.float64) * oracle.decode16(dy, act)).sum()
    assert lhs == rhs


@pytest.mark.parametrize("act", [F16, BF16])
def test_combine_adjoint_rounding_bound(act):
    """With general values dy carries one fp32 and one 16-bit rounding per
    element, so the identity holds within sum |y| |w dout| (u16 + 2^-24)."""
    T, E, k, R, H = 300, 16, 3, 4, 24
    m = layout(T, E, k, R, 7)
    rng = np.random.default_rng(8)
    y = enc(rng.standard_normal((T * k, H)), act)
    dout = enc(rng.standard_normal((T, H)), act)
    out = oracle.combine(y, m["pos"], m["w"], k, act)
    lhs = (out * oracle.decode16(dout, act).astype(np.float64)).sum()
    dy = oracle.combine_backward_dy(dout, m["src"], m["w"], k, act)
    yd = oracle.decode16(y, act).astype(np.float64)
    rhs = (yd * oracle.decode16(dy, act)).sum()
    exact = m["w"].reshape(-1)[m["src"]].astype(np.float64)[:, None] \
        * oracle.decode16(dout, act).astype(np.float64)[m["src"] // k]
    u16 = 2.0 ** -11 if act == F16 else 2.0 ** -8
    bound = (np.abs(yd) * np.abs(exact)).sum() * (u16 + 2.0 ** -24)
    assert abs(lhs - rhs) <= bound
    assert abs(lhs - rhs) > 0  # the bound is not vacuous: rounding did occur


@pytest.mark.parametrize("act", [F16, BF16])
def test_dw_is_the_derivative_in_w(act):
    """L(w) = <combine(y, w), dout> is linear in w, so L(w + e_tj) - L(w)
    equals dw[t, j] up to fp64 rounding."""
    T, E, k, R, H = 40, 8, 3, 4, 32
    m = layout(T, E, k, R, 11)
    rng = np.random.default_rng(12)
    y = enc(rng.standard_normal((T * k, H)), act)
    dout = enc(rng.standard_normal((T, H)), act)
    g = oracle.decode16(dout, act).astype(np.float64)
    w = m["w"].astype(np.float64)
    L = lambda ww: (oracle.combine(y, m["pos"], ww, k, act) * g).sum()
    dw = oracle.combine_backward_dw(y, dout, m["pos"], k, act)
    base = L(w)
    for t, j in [(0, 0), (3, 2), (17, 1), (39, 0), (39, 2)]:
        wp = w.copy()
        wp[t, j] += 1.0
        assert abs((L(wp) - base) - dw[t, j]) <= 1e-9 * (1 + abs(base))


@pytest.mark.parametrize("act", [F16, BF16])
@pytest.mark.parametrize("T,E,k,R", [(64, 8, 2, 4), (150, 16, 6, 8)])
def test_dispatch_adjoint_exact(T, E, k, R, act):
    """<dispatch(x), dsend> = <x, dx>: dx is the adjoint of the dispatch.
    Small integers keep it exact."""
    m = layout(T, E, k, R, 3 * T)
    rng = np.random.default_rng(T)
    H = 16
    x, dsend = small_ints(rng, (T, H), act), small_ints(rng, (T * k, H), act)
    send = oracle.dispatch(x, m["pos"], k)
    lhs = (oracle.decode16(send, act).astype(np.float64) * oracle.decode16(dsend, act)).sum()
    dx = oracle.dispatch_backward(dsend, m["pos"], k, act)
    rhs = (oracle.decode16(x, act).astype(np.float64) * dx).sum()
    assert lhs == rhs


def test_top1_special_case():
    """k = 1: the softmax over one logit gives w = 1, so dy is dout moved to
    the token's send row, and dx is the token's send-row gradient moved back."""
    T, E, R, H = 50, 8, 4, 8
    m = layout(T, E, 1, R, 5)
    assert (m["w"] == 1).all()
    rng = np.random.default_rng(6)
    dout = enc(rng.standard_normal((T, H)), BF16)
    dsend = enc(rng.standard_normal((T, H)), BF16)
    dy = oracle.combine_backward_dy(dout, m["src"], m["w"], 1, BF16)
    assert np.array_equal(dy[m["pos"]], dout)
    dx = oracle.dispatch_backward(dsend, m["pos"], 1, BF16)
    assert np.array_equal(dx, oracle.decode16(dsend[m["pos"]], BF16).astype(np.float64))
