"""Seeded synthetic inputs for MoE routing workloads.

Both the HIP path and the CPU oracle are fed the bytes made here; this module
draws random numbers and converts them to the storage formats and contains
none of the routing arithmetic.

Recipe (seed s, workload w):
  * three generators spawned from numpy's SeedSequence(s): logits, auxiliary
    draws (token clusters, expert permutation), activations;
  * logits: standard normal float64 [T, E], plus a per-workload bias, then one
    rounding to float32;
      - "none": no bias (the i.i.d. condition that mock-token benchmarks use);
      - "cluster_pairs": each token draws a cluster c uniformly from
        {0 .. E/2-1} and experts 2c and 2c+1 get +3.0 (experts that are often
        chosen together, as in the correlated-placement study);
      - "zipf1.2": + log p_e with p_e proportional to (e+1)^-1.2;
      - "zipf1.0_perm": a random permutation perm of the experts and
        p[perm[i]] proportional to (i+1)^-1, bias 0.5 * log p;
  * activations: standard normal float32 drawn in chunks of 4096 rows, rounded
    to nearest-even into fp16 (numpy) or bf16 (torch's CPU conversion), and
    returned as uint16 bit patterns [T, H];
  * upstream gradients for the backward (make_grad): the same row recipe from
    a fourth generator of the seed's SeedSequence (children 3 + stream), so
    they are independent of the logits and activations.
"""
from __future__ import annotations

import hashlib

import numpy as np

from .configs import BF16, F16, Workload

X_CHUNK_ROWS = 4096


def _streams(seed: int):
    ss = np.random.SeedSequence(seed)
    return [np.random.default_rng(s) for s in ss.spawn(3)]


def make_logits(w: Workload, seed: int = 0) -> np.ndarray:
    g_logit, g_aux, _ = _streams(seed)
    z = g_logit.standard_normal((w.T, w.E))
    if w.logit_bias == "cluster_pairs":
        c = g_aux.integers(0, w.E // 2, w.T)
        rows = np.arange(w.T)
        z[rows, 2 * c] += 3.0
        z[rows, 2 * c + 1] += 3.0
    elif w.logit_bias == "zipf1.2":
        p = (np.arange(w.E) + 1.0) ** -1.2
        z += np.log(p / p.sum())[None, :]
    elif w.logit_bias == "zipf1.0_perm":
        perm = g_aux.permutation(w.E)
        p = np.empty(w.E)
        p[perm] = (np.arange(w.E) + 1.0) ** -1.0
        z += 0.5 * np.log(p / p.sum())[None, :]
    elif w.logit_bias != "none":
        raise ValueError(f"unknown logit bias {w.logit_bias!r}")
    return z.astype(np.float32)


def _to_bf16_bits(f32: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(f32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _rows16(g: np.random.Generator, n: int, H: int, act_dtype: int) -> np.ndarray:
    out = np.empty((n, H), dtype=np.uint16)
    for r0 in range(0, n, X_CHUNK_ROWS):
        rows = min(X_CHUNK_ROWS, n - r0)
        f = g.standard_normal((rows, H), dtype=np.float32)
        if act_dtype == F16:
            out[r0:r0 + rows] = f.astype(np.float16).view(np.uint16)
        elif act_dtype == BF16:
            out[r0:r0 + rows] = _to_bf16_bits(f)
        else:
            raise ValueError("act_dtype")
    return out


def make_x(w: Workload, seed: int = 0) -> np.ndarray:
    _, _, g_x = _streams(seed)
    return _rows16(g_x, w.T, w.H, w.act_dtype)


def make_grad(w: Workload, seed: int, rows: int, stream: int = 0) -> np.ndarray:
    """Seeded upstream-gradient rows [rows, H] as uint16 bit patterns."""
    g = np.random.default_rng(np.random.SeedSequence(seed).spawn(4 + stream)[3 + stream])
    return _rows16(g, rows, w.H, w.act_dtype)


def digest(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).view(np.uint8)).hexdigest()[:16]
