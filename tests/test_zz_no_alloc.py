"""moe_route_assign_layout_noalloc, the route + assignment + layout call that
allocates nothing (its scratch is a static device array): its outputs equal,
bit for bit, those of moe_route_assign_layout with a caller-allocated
workspace, on consecutive calls through the C ABI, each smaller than the one
before, so the static scratch is reused with the previous call's contents
left in it. Also the host-side rejection of problems whose tables do not fit
the static scratch."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from combine_router_topk_amd import binding as B
from combine_router_topk_amd import path as P

OUTPUTS = ("idx", "w", "counts", "assign", "active", "rank_of", "expert_offsets", "rank_offsets",
           "pos", "src", "dedup")


def say(msg):
    print(msg, flush=True)


def outputs_like(b):
    return {name: torch.full_like(getattr(b, name).view(torch.int32) if getattr(b, name).dtype == torch.float32
                                  else getattr(b, name), -7)
            for name in OUTPUTS}


def noalloc(b, o):
    B.moe_route_assign_layout_noalloc(b.p, b.logits, b.rep, b.maxrep, o["idx"], o["w"].view(torch.float32),
                                      o["counts"], o["assign"], o["active"], o["rank_of"],
                                      o["expert_offsets"], o["rank_offsets"], o["pos"], o["src"],
                                      o["dedup"])


CASES = [  # each smaller than the one before; the first two take the multi-launch path
    synth.TRAIN_TOP2,
    synth.scaled(synth.LARGE, T=3000, H=8),
    synth.DECODE,
    synth.TINY,
]


@pytest.mark.gpu
def test_noalloc_equals_workspace_call_on_consecutive_shrinking_calls():
    for i, w in enumerate(CASES):
        say(f"[case] no-alloc call {i}: {w.name} T={w.T} E={w.E} k={w.k} R={w.R}")
        p = B.make_problem(w.T, w.E, w.k, 8, w.R, w.act_dtype)
        logits = synth.make_logits(w, i)
        rep = synth.replica_table(w)
        x = torch.zeros(w.T, 8, dtype=torch.float16 if w.act_dtype == synth.F16 else torch.bfloat16)
        b = P.allocate(p, torch.from_numpy(logits), x, None if rep is None else torch.from_numpy(rep))
        P.route_assign_layout(b)
        o = outputs_like(b)
        noalloc(b, o)
        torch.cuda.synchronize()
        for name in OUTPUTS:
            want = getattr(b, name)
            want = want.view(torch.int32) if want.dtype == torch.float32 else want
            assert torch.equal(o[name], want), (w.name, name)


def test_noalloc_rejects_problems_beyond_the_static_scratch():
    """Checked on the host before anything is enqueued or any device is
    touched: E + R above 1024 with enough tokens needs more than 2 MiB of
    route rows (512 blocks of E + R counts). (The
    pointers are never dereferenced: the call returns at the size check.)"""
    for T, E, R in ((8192, 1024, 8), (1 << 16, 1024, 64)):
        p = B.make_problem(T, E, 8, 8, R, B.MOE_BF16)
        fake = ctypes.c_void_p(1 << 20)
        st = B._lib.moe_route_assign_layout_noalloc(ctypes.byref(p), fake, None, 1, *([fake] * 11), None)
        assert st == B.MOE_ERR_WORKSPACE, (T, E, R)
        assert "static scratch" in B.moe_last_error()
