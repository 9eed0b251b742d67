"""Row movement: dispatch into send rows, the expert stand-in, and the
weighted combine back to token order (oracle).

Sources:
  * "METRO AllGather vs AllToAll for MoE decode", section "Work the 8-GPU
    payload example": the dispatch payload is token activation rows; section
    "METRO AllGather vs AllToAll changes the routing information": expert
    outputs come back to their tokens through a combine.
  * News summary of correlated expert placement and token shuffling, section
    "Why communication is the target": each MoE layer dispatches tokens and
    combines results.

Activations are 16-bit floats (fp16 or bf16) held as uint16 bit patterns.
"""
from __future__ import annotations

import numpy as np

F16 = 1
BF16 = 2


def decode16(bits: np.ndarray, act_dtype: int) -> np.ndarray:
    """uint16 bit patterns -> float32 values (exact)."""
    bits = np.asarray(bits, dtype=np.uint16)
    if act_dtype == F16:
        return bits.view(np.float16).astype(np.float32)
    if act_dtype == BF16:
        return (bits.astype(np.uint32) << 16).view(np.float32)
    raise ValueError("act_dtype")


def encode16(f32: np.ndarray, act_dtype: int) -> np.ndarray:
    """float32 -> uint16 bit patterns, rounding to nearest, ties to even."""
    f32 = np.asarray(f32, dtype=np.float32)
    if act_dtype == F16:
        return f32.astype(np.float16).view(np.uint16)
    if act_dtype == BF16:
        u = f32.view(np.uint32).astype(np.uint64)
        r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
        nan = np.isnan(f32)
        if nan.any():
            r[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
        return r
    raise ValueError("act_dtype")


def dispatch(x: np.ndarray, pos: np.ndarray, k: int) -> np.ndarray:
    """send[pos[i]] = x[i // k]: a bit copy of token rows into send rows.
    [T*k, H] uint16."""
    n = pos.shape[0]
    send = np.empty((n, x.shape[1]), dtype=x.dtype)
    send[pos] = x[np.arange(n) // k]
    return send


def dispatch_rows(x: np.ndarray, src: np.ndarray, k: int, rows: np.ndarray) -> np.ndarray:
    """The same copy for selected send rows only: send[r] = x[src[r] // k]."""
    return x[np.asarray(src)[rows] // k]


def expert_standin(send_rows: np.ndarray, row_experts: np.ndarray, E: int, act_dtype: int) -> np.ndarray:
    """Stand-in for the expert computation (the pages' expert GEMMs need
    trained weights): y = x * (1 + e/E) for a row routed to expert e.
    Precision fixed by the workload: scale = 1 + e/E and the product are each
    rounded to fp32, the product then to the 16-bit activation format (for E
    a power of two both fp32 results are exact, so y is x*(1+e/E) rounded
    once)."""
    e = np.asarray(row_experts).astype(np.float32)
    scale = np.float32(1.0) + e / np.float32(E)
    prod = decode16(send_rows, act_dtype) * scale[:, None]
    return encode16(prod, act_dtype)


def combine(y: np.ndarray, pos: np.ndarray, w: np.ndarray, k: int, act_dtype: int,
            tokens: np.ndarray | None = None) -> np.ndarray:
    """out[t] = sum over slots j ascending of w[t, j] * y[pos[t*k + j]],
    evaluated in fp64. Returns float64 [len(tokens), H]."""
    T = w.shape[0]
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    acc = np.zeros((tokens.shape[0], y.shape[1]), dtype=np.float64)
    for j in range(k):
        rows = np.asarray(pos)[tokens * k + j]
        acc = acc + np.asarray(w)[tokens, j].astype(np.float64)[:, None] \
            * decode16(y[rows], act_dtype).astype(np.float64)
    return acc
