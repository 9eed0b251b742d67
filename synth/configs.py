"""Workload shapes for MoE token routing on one GPU.

Each workload is one GPU's share of an expert-parallel MoE layer: T tokens,
E experts, top-k routing, hidden width H, activations in a 16-bit float
format, and R virtual expert-parallel ranks that exist only as a layout
inside one GPU's memory.

Sources of the shapes:
  * "METRO AllGather vs AllToAll for MoE decode", section "Work the 8-GPU
    payload example": 32 decode tokens per GPU on 8 GPUs, fp16, hidden 4096
    (the decode workload below).
  * The news summary of correlated expert placement and token shuffling,
    section "Why communication is the target": expert-parallel degree 32 with
    top-2 and top-6 routing on MI300X nodes (the two training workloads).
  * "Diagnosing Overhead in Dispatch Operations: Cross-architecture
    Observatory", section "Key Findings": some architectures keep routing
    concentrated on a few experts (the two skewed workloads).

This module holds shapes and replica tables only; it contains none of the
routing arithmetic.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

F16 = 1
BF16 = 2
DTYPE_NAMES = {F16: "f16", BF16: "bf16"}


@dataclass(frozen=True)
class Workload:
    name: str
    T: int            # tokens
    E: int            # experts
    k: int            # experts selected per token
    H: int            # hidden width (elements per activation row)
    R: int            # virtual expert-parallel ranks (= virtual GPUs)
    act_dtype: int    # F16 or BF16
    logit_bias: str   # "none" | "cluster_pairs" | "zipf1.2" | "zipf1.0_perm"
    replicated: bool  # True: the decode replica table below

    @property
    def row_bytes(self) -> int:
        return self.H * 2

    @property
    def dtype_name(self) -> str:
        return DTYPE_NAMES[self.act_dtype]

    def dispatch_combine_bytes(self) -> int:
        """Bytes the dispatch and combine must move: dispatch reads each token
        row once and writes k copies; combine reads k rows and writes one."""
        return 2 * (1 + self.k) * self.T * self.H * 2


WORKLOADS = [
    Workload("tiny_T256_E8_k2_H128_f16", 256, 8, 2, 128, 4, F16, "none", False),
    Workload("decode_T256_E256_k8_H4096_f16_replicated", 256, 256, 8, 4096, 8, F16, "none", True),
    Workload("train_T16384_E64_k2_H4096_bf16_clustered", 16384, 64, 2, 4096, 32, BF16, "cluster_pairs", False),
    Workload("train_T16384_E64_k6_H2048_bf16_zipf", 16384, 64, 6, 2048, 64, BF16, "zipf1.2", False),
    Workload("large_T65536_E256_k8_H7168_bf16_zipf", 65536, 256, 8, 7168, 32, BF16, "zipf1.0_perm", False),
]
BY_NAME = {w.name: w for w in WORKLOADS}
TINY, DECODE, TRAIN_TOP2, TRAIN_TOP6, LARGE = WORKLOADS


def replica_table(w: Workload) -> np.ndarray | None:
    """int32 [E, maxrep] table of virtual-GPU ids that hold a copy of each
    expert, -1 padded, column 0 the primary copy; None for the plain
    contiguous partition (expert e lives on rank e // (E / R)).

    Decode table: expert e's primary copy is on GPU e // (E / R); every
    eighth expert (e % 8 == 0) has a second copy on GPU (e // (E/R) + R/2) % R.
    With E=256, R=8 that is 32 replicated experts (1.125x replication)."""
    if not w.replicated:
        return None
    per = w.E // w.R
    rep = np.full((w.E, 2), -1, dtype=np.int32)
    for e in range(w.E):
        rep[e, 0] = e // per
        if e % 8 == 0:
            rep[e, 1] = (e // per + w.R // 2) % w.R
    return rep


def scaled(w: Workload, T: int | None = None, H: int | None = None, name: str | None = None) -> Workload:
    """Same routing structure at another token count or hidden width (used by
    tests for small cases with several tiles and a ragged tail)."""
    T = w.T if T is None else T
    H = w.H if H is None else H
    return Workload(name or f"{w.name}@T{T}H{H}", T, w.E, w.k, H, w.R, w.act_dtype,
                    w.logit_bias, w.replicated)
