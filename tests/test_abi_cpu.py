"""The C-ABI library without a GPU: it loads, exports every entry point that
include/moe_route.h declares, and its host-side checks turn bad arguments
into status codes before anything is enqueued (no compute calls here)."""
import ctypes
import os
import re

import pytest

from conftest import ROOT
from combine_router_topk_amd import binding as B

HEADER = os.path.join(ROOT, "include", "moe_route.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_header_declares_and_library_exports_every_entry_point():
    names = declared_functions()
    assert set(names) == set(B.EXPORTED), names
    lib = ctypes.CDLL(B.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_build_id_is_the_digest_of_the_sources_and_a_mismatch_is_refused(monkeypatch):
    from combine_router_topk_amd import build
    bid = B.moe_build_id()
    assert len(bid) == 16 and int(bid, 16) >= 0
    assert bid == build.source_digest()
    monkeypatch.setattr(build, "source_digest", lambda: "0" * 16)
    with pytest.raises(ImportError, match="other sources"):
        B._load()


def test_source_digest_covers_every_source_and_header():
    from combine_router_topk_amd import build
    names = {os.path.relpath(f, ROOT) for f in build.source_files()}
    assert "include/moe_route.h" in names
    csrc = os.path.join(ROOT, "combine_router_topk_amd", "csrc")
    for f in os.listdir(csrc):
        if f.endswith((".hip", ".hpp")):
            assert os.path.join("combine_router_topk_amd", "csrc", f) in names, f


def test_version_and_status_strings():
    assert B.moe_version() >= 10000
    assert B.moe_status_string(0) == "ok"
    assert B.moe_status_string(3) == "workspace too small"
    assert B.moe_status_string(99) == "unknown status"


def prob(**kw):
    d = dict(T=256, E=8, k=2, H=128, R=4, act_dtype=B.MOE_F16, flags=0)
    d.update(kw)
    return B.make_problem(d["T"], d["E"], d["k"], d["H"], d["R"], d["act_dtype"], d["flags"])


@pytest.mark.parametrize("bad", [dict(T=-1), dict(E=0), dict(E=1025), dict(k=0), dict(k=9),
                                 dict(E=32, k=17), dict(H=12), dict(H=0), dict(R=0),
                                 dict(R=1025), dict(act_dtype=3), dict(flags=1 << 7),
                                 dict(T=1 << 30, k=4), dict(T=1 << 23, k=2)])
def test_invalid_problems_rejected(bad):
    n = ctypes.c_size_t(0)
    st = B._lib.moe_workspace_bytes(ctypes.byref(prob(**bad)), ctypes.byref(n))
    assert st == B.MOE_ERR_INVALID_ARG, (bad, B.moe_last_error())
    assert B.moe_last_error()


def test_row_limit_is_inclusive():
    """T*k up to 2^24 - 1 is accepted: a one-block-per-row launch of that many
    256-thread blocks stays under 2^32 work-items."""
    n = ctypes.c_size_t(0)
    for T, k in (((1 << 24) - 1, 1), ((1 << 23) - 1, 2)):
        assert B._lib.moe_workspace_bytes(ctypes.byref(prob(T=T, k=k)), ctypes.byref(n)) == B.MOE_OK
        assert n.value > 0


def test_workspace_size_grows_with_tokens():
    sizes = [B.moe_workspace_bytes(prob(T=t, E=64, R=32)) for t in (0, 1, 1000, 16384, 65536)]
    assert all(s % 256 == 0 and s > 0 for s in sizes)
    assert sizes == sorted(sizes)


def test_null_pointers_rejected_before_any_launch():
    p = prob()
    ref = ctypes.byref(p)
    lib = B._lib
    fake = ctypes.c_void_p(1 << 20)           # aligned, never dereferenced
    mis = ctypes.c_void_p((1 << 20) + 4)      # 4-byte aligned, not 16
    assert lib.moe_route(ref, None, fake, fake, fake, fake, 1 << 20, None) == B.MOE_ERR_INVALID_ARG
    assert "logits" in B.moe_last_error()
    assert lib.moe_route(ref, fake, fake, fake, fake, fake, 16, None) == B.MOE_ERR_WORKSPACE
    assert lib.moe_assign_replicas(ref, fake, None, 1, None, fake, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_assign_replicas(ref, fake, fake, 0, fake, fake, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_layout(ref, fake, None, None, 1, fake, fake, fake, None, fake, fake, fake,
                          1 << 20, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_dispatch(ref, mis, fake, fake, None) == B.MOE_ERR_INVALID_ARG
    assert "aligned" in B.moe_last_error()
    assert lib.moe_expert_standin(ref, fake, fake, fake, None, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_combine(ref, fake, fake, None, fake, None) == B.MOE_ERR_INVALID_ARG
    # no replica table: R must divide E
    p2 = prob(E=12, R=5)
    assert lib.moe_assign_replicas(ctypes.byref(p2), fake, None, 1, fake, fake, None) \
        == B.MOE_ERR_INVALID_ARG


def test_empty_rows_are_noops():
    p = prob(T=0)
    ref = ctypes.byref(p)
    assert B._lib.moe_dispatch(ref, None, None, None, None) == B.MOE_OK
    assert B._lib.moe_expert_standin(ref, None, None, None, None, None) == B.MOE_OK
    assert B._lib.moe_combine(ref, None, None, None, None, None) == B.MOE_OK


def test_product_path_never_touches_the_oracle():
    pkg = os.path.join(ROOT, "combine_router_topk_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"\boracle\b", text), f


def test_new_entry_points_reject_bad_arguments_before_any_launch():
    p = prob()
    ref = ctypes.byref(p)
    lib = B._lib
    fake = ctypes.c_void_p(1 << 20)
    mis = ctypes.c_void_p((1 << 20) + 4)
    ws = 1 << 20
    # single-send layout: a NULL single-send output, a short workspace
    assert lib.moe_layout_single_send(ref, fake, None, None, 1, fake, fake, fake, fake, fake, fake,
                                      None, fake, fake, fake, ws, None) == B.MOE_ERR_INVALID_ARG
    assert "ss_rank_offsets" in B.moe_last_error()
    assert lib.moe_layout_single_send(ref, fake, None, None, 1, fake, fake, fake, fake, fake, fake,
                                      fake, fake, fake, fake, 16, None) == B.MOE_ERR_WORKSPACE
    # single-send dispatch and fan-out: negative capacity, misaligned rows
    assert lib.moe_single_send_dispatch(ref, fake, fake, fake, -1, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_single_send_dispatch(ref, mis, fake, fake, 8, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_single_send_expand(ref, fake, fake, fake, fake, fake, -1, fake, None) \
        == B.MOE_ERR_INVALID_ARG
    assert lib.moe_single_send_expand(ref, fake, None, fake, fake, fake, 8, fake, None) \
        == B.MOE_ERR_INVALID_ARG
    # capacity 0 and T = 0 are no-ops
    assert lib.moe_single_send_dispatch(ref, None, None, None, 0, None) == B.MOE_OK
    # backward: both outputs NULL, y missing for dw, w missing for dy
    assert lib.moe_combine_backward(ref, fake, fake, fake, fake, None, None, None) \
        == B.MOE_ERR_INVALID_ARG
    assert lib.moe_combine_backward(ref, fake, None, fake, fake, None, fake, None) \
        == B.MOE_ERR_INVALID_ARG
    assert "y" in B.moe_last_error()
    assert lib.moe_combine_backward(ref, fake, fake, fake, None, fake, None, None) \
        == B.MOE_ERR_INVALID_ARG
    assert lib.moe_dispatch_backward(ref, fake, fake, mis, None) == B.MOE_ERR_INVALID_ARG
    # statistics: the f64 output is required and 8-byte aligned
    assert lib.moe_routing_stats(ref, fake, fake, fake, fake, None, None, None) \
        == B.MOE_ERR_INVALID_ARG
    assert lib.moe_routing_stats(ref, fake, fake, fake, fake, None, mis, None) \
        == B.MOE_ERR_INVALID_ARG
    # token-balanced split: no table needs R | E; a table needs 1 <= maxrep <= 16
    p2 = prob(E=12, R=5)
    assert lib.moe_token_balanced_split(ctypes.byref(p2), fake, fake, fake, fake, None, 1, fake,
                                        fake, fake, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_token_balanced_split(ref, fake, fake, fake, fake, fake, 17, fake, fake, fake,
                                        None) == B.MOE_ERR_INVALID_ARG


def test_new_entry_points_empty_batch_is_noop_where_nothing_is_written():
    p = prob(T=0)
    ref = ctypes.byref(p)
    lib = B._lib
    assert lib.moe_single_send_dispatch(ref, None, None, None, 4, None) == B.MOE_OK
    assert lib.moe_single_send_expand(ref, None, None, None, None, None, 4, None, None) == B.MOE_OK
    assert lib.moe_combine_backward(ref, None, None, None, None, None, None, None) == B.MOE_OK
    assert lib.moe_dispatch_backward(ref, None, None, None, None) == B.MOE_OK


def test_plain_c_caller_builds_and_exports_its_check():
    from conftest import C_CHECK_LIB
    lib = ctypes.CDLL(C_CHECK_LIB)
    assert hasattr(lib, "moe_c_abi_check") and hasattr(lib, "moe_c_abi_check_rest")


def test_plain_c_caller_calls_every_compute_entry_point():
    """Every call of the header that enqueues work is made from plain C."""
    header = open(HEADER).read()
    calls = set(re.findall(r"^moe_status (moe_\w+)\(", header, re.M)) - {"moe_workspace_bytes"}
    assert len(calls) >= 16
    src = open(os.path.join(ROOT, "tests", "c_abi", "check_abi.c")).read()
    missing = sorted(c for c in calls if not re.search(rf"\b{c}\(", src))
    assert not missing, missing


def test_binding_limits_match_header():
    text = open(HEADER).read()
    for name in ("MOE_MAX_E", "MOE_MAX_K", "MOE_MAX_R", "MOE_MAX_REP"):
        m = re.search(rf"{name} = (\d+)", text)
        assert m and int(m.group(1)) == getattr(B, name), name
    assert "MOE_MAX_ROWS = (1 << 24) - 1" in text and B.MOE_MAX_ROWS == (1 << 24) - 1


def test_binding_hands_missing_buffers_to_the_library_checks():
    # a missing workspace or buffer reaches the library as NULL with 0 bytes,
    # and comes back as a MoeError naming it (stream 0: nothing is enqueued)
    p = B.make_problem(4, 8, 2, 64, 4, B.MOE_BF16)
    with pytest.raises(B.MoeError, match="counts is NULL") as e:
        B.moe_route(p, None, None, None, None, None, stream=0)
    assert e.value.status == B.MOE_ERR_INVALID_ARG
    with pytest.raises(B.MoeError, match="is NULL"):
        B.moe_layout(p, None, None, None, 1, *(None,) * 7, stream=0)
    with pytest.raises(B.MoeError, match="is NULL"):
        B.moe_layout_single_send(p, None, None, None, 1, *(None,) * 10, stream=0)
    # a single-send buffer of no rows has capacity 0: nothing is written
    B.moe_single_send_dispatch(p, None, None, None, stream=0)
    B.moe_single_send_expand(p, *(None,) * 6, stream=0)


def test_route_assign_layout_rejects_bad_arguments_before_any_launch():
    p = prob()
    ref = ctypes.byref(p)
    lib = B._lib
    fake = ctypes.c_void_p(1 << 20)
    ws = 1 << 20

    def call(logits=fake, rep=None, maxrep=1, idx=fake, w=fake, counts=fake, assign=fake,
             active=fake, rank_of=fake, eo=fake, ro=fake, pos=fake, src=fake, dedup=fake,
             wsp=fake, wsb=ws, pp=ref):
        return lib.moe_route_assign_layout(pp, logits, rep, maxrep, idx, w, counts, assign, active,
                                           rank_of, eo, ro, pos, src, dedup, wsp, wsb, None)
    for field in ("logits", "idx", "w", "counts", "assign", "active", "rank_of", "pos", "src",
                  "dedup"):
        assert call(**{field: None}) == B.MOE_ERR_INVALID_ARG, field
        assert field in B.moe_last_error()
    assert call(eo=None) == B.MOE_ERR_INVALID_ARG and "expert_offsets" in B.moe_last_error()
    assert call(ro=None) == B.MOE_ERR_INVALID_ARG and "rank_offsets" in B.moe_last_error()
    assert call(wsp=None) == B.MOE_ERR_INVALID_ARG and "ws" in B.moe_last_error()
    assert call(wsb=16) == B.MOE_ERR_WORKSPACE
    assert call(rep=fake, maxrep=0) == B.MOE_ERR_INVALID_ARG and "maxrep" in B.moe_last_error()
    p2 = prob(E=12, R=5)  # no replica table: R must divide E
    assert call(pp=ctypes.byref(p2)) == B.MOE_ERR_INVALID_ARG
    # an empty batch needs no logits, idx, w, pos or src (nothing is launched here:
    # the workspace size is checked first and is too small)
    p0 = prob(T=0)
    assert call(pp=ctypes.byref(p0), logits=None, idx=None, w=None, pos=None, src=None,
                wsb=0) == B.MOE_ERR_WORKSPACE
