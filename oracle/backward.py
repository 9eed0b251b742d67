"""Backward of the row movement (oracle): the gradients of the combine with
respect to the expert outputs and to the gate weights, and of the dispatch
with respect to the token rows.

Source: news summary of correlated expert placement and token shuffling,
section "Why communication is the target" (every MoE layer dispatches tokens
and combines results in the forward and again in the backward pass).

The pages print no formulas for the backward; the gradients below follow
from the forward definitions by differentiation. The forward maps are

    combine:  out[t] = sum_j w[t, j] * y[pos[t*k + j]]
    dispatch: send[pos[i]] = x[i // k]

so, for an upstream gradient dout [T, H] of out and dsend [T*k, H] of send:

    dy[pos[t*k + j]] = w[t, j] * dout[t]                 (a weighted scatter)
    dw[t, j]         = <y[pos[t*k + j]], dout[t]>        (a row dot product)
    dx[t]            = sum_j dsend[pos[t*k + j]]          (an unweighted gather-sum)

Readings (the pages fix no precision): dy is the fp32 product of the fp32
gate weight and the 16-bit gradient, rounded once to the activation format,
like the forward's row outputs; dw and dx are exact sums here (fp64 over
products that are exact), which a kernel's fp32 sums are compared against
within their rounding bound.

Activations and gradients are 16-bit floats held as uint16 bit patterns.
"""
from __future__ import annotations

import numpy as np

from .rows import decode16, encode16


def combine_backward_dy(dout: np.ndarray, src: np.ndarray, w: np.ndarray, k: int, act_dtype: int,
                        rows: np.ndarray | None = None) -> np.ndarray:
    """dy for send rows `rows` (all when None): row r carries pair i = src[r]
    of token i // k and slot i % k, so dy[r] = rne16(f32(w[i]) * f32(dout[i // k])).
    uint16 [len(rows), H]."""
    src = np.asarray(src)
    rows = np.arange(src.shape[0]) if rows is None else np.asarray(rows)
    pair = src[rows]
    wf = np.asarray(w, dtype=np.float32).reshape(-1)[pair]
    prod = wf[:, None] * decode16(dout[pair // k], act_dtype)  # fp32 product, rounded once
    return encode16(prod, act_dtype)


def combine_backward_dw(y: np.ndarray, dout: np.ndarray, pos: np.ndarray, k: int, act_dtype: int,
                        tokens: np.ndarray | None = None) -> np.ndarray:
    """dw[t, j] = <y[pos[t*k + j]], dout[t]> in fp64 for the chosen tokens.
    float64 [len(tokens), k]."""
    T = dout.shape[0]
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    pos = np.asarray(pos)
    g = decode16(dout[tokens], act_dtype).astype(np.float64)
    dw = np.empty((tokens.shape[0], k), dtype=np.float64)
    for j in range(k):
        yr = decode16(y[pos[tokens * k + j]], act_dtype).astype(np.float64)
        dw[:, j] = (yr * g).sum(axis=1)
    return dw


def dispatch_backward(dsend: np.ndarray, pos: np.ndarray, k: int, act_dtype: int,
                      tokens: np.ndarray | None = None, T: int | None = None) -> np.ndarray:
    """dx[t] = sum over slots j of dsend[pos[t*k + j]] in fp64 for the chosen
    tokens. float64 [len(tokens), H]."""
    pos = np.asarray(pos)
    T = pos.shape[0] // k if T is None else T
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    acc = np.zeros((tokens.shape[0], dsend.shape[1]), dtype=np.float64)
    for j in range(k):
        acc = acc + decode16(dsend[pos[tokens * k + j]], act_dtype).astype(np.float64)
    return acc
