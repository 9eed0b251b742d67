"""Payload byte model of the two dispatch collectives (oracle).

Source: "METRO AllGather vs AllToAll for MoE decode", section "Work the 8-GPU
payload example" (per-GPU payload of an all-to-all dispatch against an
all-gather of every rank's tokens, and its ideal link time) and section "Find
the crossover instead of copying 2 MB" (the payload whose ideal link time
equals a fixed collective latency).

Reading taken: the all-to-all figure counts one copy of each local token row
per GPU, and the all-gather figure every rank's token rows; the page's byte
figures use binary prefixes (KB = 2^10 B, MB = 2^20 B).
"""
from __future__ import annotations


def alltoall_bytes_per_gpu(tokens_per_gpu: int, hidden: int, elem_bytes: int) -> int:
    return tokens_per_gpu * hidden * elem_bytes


def allgather_bytes_per_gpu(tokens_per_gpu: int, gpus: int, hidden: int, elem_bytes: int) -> int:
    return tokens_per_gpu * gpus * hidden * elem_bytes


def link_time_s(nbytes: float, bytes_per_s: float) -> float:
    return nbytes / bytes_per_s


def crossover_bytes(latency_s: float, bytes_per_s: float) -> float:
    return latency_s * bytes_per_s
