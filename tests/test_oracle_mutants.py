"""The oracle's pins against planted mistakes: each case replaces one oracle
function with a plausible wrong version (a flipped tie rule, a dropped term,
a transposed order, an off-by-one) in every oracle module that binds it, and
runs the pins that should notice. At least one of them must fail, so the
pins are shown to separate the oracle from its likely mistakes rather than
to agree with it by construction (no GPU; the mistakes live only here)."""
import sys

import numpy as np
import pytest

import oracle
import oracle.eplb
import oracle.stats
import test_oracle_eplb as TE
import test_oracle_layout as TL
import test_oracle_replicas as TP
import test_oracle_route as TR
import test_oracle_rows as TW
import test_oracle_single_send as TS
import test_oracle_stats as TT
from oracle.rows import BF16

O = {name: getattr(oracle, name) for name in (
    "topk_select", "gate_weights", "demand_vector", "greedy_assign", "permutation", "expert_ranks",
    "segment_offsets", "dedup_counts", "encode16", "expert_standin", "combine",
    "single_send_layout", "gini", "coselection", "routing_stats")}
O["replica_share_index"] = oracle.eplb.replica_share_index


def plant(monkeypatch, name, fn):
    """Binds `fn` under `name` in the package and in every oracle module."""
    mods = [m for k, m in sys.modules.items() if k == "oracle" or k.startswith("oracle.")]
    hit = 0
    for m in mods:
        if hasattr(m, name):
            monkeypatch.setattr(m, name, fn)
            hit += 1
    assert hit > 0, name


def some_pin_fails(pins):
    failed = []
    for pin, args in pins:
        try:
            pin(*args)
        except AssertionError:
            failed.append(pin.__name__)
    return failed


# ---- the planted mistakes ----------------------------------------------------

def topk_ties_to_higher_id(l, k):
    E = l.shape[1]
    return (E - 1 - O["topk_select"](np.ascontiguousarray(l[:, ::-1]), k)).astype(np.int32)


def topk_minus_zero_below_plus_zero(l, k):
    l2 = np.array(l, np.float32, copy=True)
    l2[(l2 == 0) & np.signbit(l2)] = np.float32(-1e-45)
    return O["topk_select"](l2, k)


def weights_over_every_expert(l, idx):
    l64 = np.asarray(l, np.float64)
    e = np.exp(l64 - l64.max(axis=1, keepdims=True))
    return (np.take_along_axis(e, np.asarray(idx), 1) / e.sum(axis=1, keepdims=True)).astype(np.float32)


def demand_drops_last_slot(idx, E):
    return O["demand_vector"](np.asarray(idx)[:, :-1], E)


def greedy_ties_to_higher_gpu(counts, R, rep, order="constrained"):
    if rep is None:
        return O["greedy_assign"](counts, R, rep, order)
    rev = np.where(rep >= 0, R - 1 - rep, rep).astype(np.int32)
    a, act = O["greedy_assign"](counts, R, rev, order)
    return np.where(a >= 0, R - 1 - a, a).astype(a.dtype), act[::-1].copy()


def greedy_ties_to_first_listed_replica(counts, R, rep, order="constrained"):
    """Fewest activated experts, ties to the earlier replica slot rather than
    the lower GPU index."""
    counts = np.asarray(counts)
    E = counts.shape[0]
    cand = oracle.candidates(E, R, rep)
    live = [e for e in range(E) if counts[e] > 0]
    if order == "constrained":
        live.sort(key=lambda e: (len(cand[e]), e))
    active, assign = [0] * R, [-1] * E
    for e in live:
        slot = min(range(len(cand[e])), key=lambda s: (active[cand[e][s]], s))
        assign[e] = cand[e][slot]
        active[assign[e]] += 1
    return np.array(assign, dtype=np.int32), np.array(active, dtype=np.int32)


def inactive_experts_on_last_copy(E, R, rep, assign):
    cand = oracle.candidates(E, R, rep)
    primary = np.array([c[0] for c in cand], dtype=np.int32)
    if assign is None:
        return primary
    last = np.array([c[-1] for c in cand], dtype=np.int32)
    assign = np.asarray(assign)
    return np.where(assign >= 0, assign, last).astype(np.int32)


def greedy_always_id_order(counts, R, rep, order="constrained"):
    return O["greedy_assign"](counts, R, rep, "id")


def permutation_tokens_descending(idx, rank_of):
    idx = np.asarray(idx)
    T, k = idx.shape
    p2, _ = O["permutation"](np.ascontiguousarray(idx[::-1]), rank_of)
    t = np.repeat(np.arange(T), k)
    j = np.tile(np.arange(k), T)
    pos = p2[(T - 1 - t) * k + j].astype(np.int32)
    src = np.empty_like(pos)
    src[pos] = np.arange(T * k, dtype=np.int32)
    return pos, src


def offsets_inclusive(counts, rank_of, R):
    eo, ro = O["segment_offsets"](counts, rank_of, R)
    return (eo + np.asarray(counts)).astype(eo.dtype), ro


def dedup_counts_pairs(idx, rank_of, R):
    return np.bincount(np.asarray(rank_of)[np.asarray(idx)].ravel(), minlength=R).astype(np.int32)


def encode16_truncates(f32, act_dtype):
    if act_dtype != BF16:
        return O["encode16"](f32, act_dtype)
    return (np.asarray(f32, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def standin_expert_off_by_one(send_rows, row_experts, E, act_dtype):
    return O["expert_standin"](send_rows, np.asarray(row_experts) + 1, E, act_dtype)


def combine_unit_weight_slot0(y, pos, w, k, act_dtype, tokens=None):
    w2 = np.array(w, np.float32, copy=True)
    w2[:, 0] = 1.0
    return O["combine"](y, pos, w2, k, act_dtype, tokens)


def single_send_token_major(idx, rank_of, R):
    idx = np.asarray(idx)
    T, k = idx.shape
    ranks = np.asarray(rank_of)[idx]
    pairs = sorted({(t, int(ranks[t, j])) for t in range(T) for j in range(k)})
    row_of = {p: q for q, p in enumerate(pairs)}
    ss_row = np.array([row_of[(t, int(ranks[t, j]))] for t in range(T) for j in range(k)], np.int32)
    ss_token = np.array([t for t, _ in pairs], np.int32)
    per_rank = np.bincount(np.array([r for _, r in pairs], np.int64), minlength=R)
    return np.concatenate([[0], np.cumsum(per_rank)]).astype(np.int32), ss_row, ss_token


def gini_doubled(loads):
    return 2.0 * O["gini"](loads)


def coselection_both_triangles(idx, E):
    C = O["coselection"](idx, E)
    return C + C.T


def locality_off_diagonal(idx, counts, rank_of, E, R):
    S, C, st = O["routing_stats"](idx, counts, rank_of, E, R)
    st = st.copy()
    st[3] = 1.0 - st[3]
    return S, C, st


def shares_larger_last(i, n, m):
    return m - 1 - O["replica_share_index"](n - 1 - i, n, m)


CASES = [
    ("topk ties to the higher id", "topk_select", topk_ties_to_higher_id,
     [(TR.test_topk_signed_zero_tie_goes_to_lower_id, ()),
      (TR.test_topk_brute_force_with_ties_zeros_nan, (0, 8, 2))]),
    ("topk -0 below +0", "topk_select", topk_minus_zero_below_plus_zero,
     [(TR.test_topk_signed_zero_tie_goes_to_lower_id, ()),
      (TR.test_topk_brute_force_with_ties_zeros_nan, (0, 8, 2))]),
    ("softmax over every expert", "gate_weights", weights_over_every_expert,
     [(TR.test_weights_top2_closed_form, ()), (TR.test_weights_top1_is_one_and_sums_to_one, ())]),
    ("demand vector drops the last slot", "demand_vector", demand_drops_last_slot,
     [(TR.test_demand_vector_bruteforce_and_sum, (0,)), (TR.test_handworked_topk_and_counts, ())]),
    ("greedy ties to the higher GPU", "greedy_assign", greedy_ties_to_higher_gpu,
     [(TP.test_handworked_replicated_instances, ()),
      (TP.test_decode_table_all_active_closed_form, ("id", "active_id_order"))]),
    ("greedy ties to the first-listed replica", "greedy_assign", greedy_ties_to_first_listed_replica,
     [(TP.test_decode_table_all_active_full_assignment, ("constrained", "two_copy_assign_constrained_order")),
      (TP.test_handworked_ties_go_to_the_lower_gpu_not_the_first_slot, ()),
      (TP.test_greedy_matches_scan_reimplementation_on_shuffled_slots, (0,)),
      (TP.test_greedy_does_not_depend_on_replica_slot_order, (0,))]),
    ("greedy ignores the most-constrained order", "greedy_assign", greedy_always_id_order,
     [(TP.test_decode_table_all_active_closed_form, ("constrained", "active_constrained_order"))]),
    ("inactive experts on their last-listed copy", "expert_ranks", inactive_experts_on_last_copy,
     [(TL.test_inactive_experts_sit_on_their_first_listed_copy, ())]),
    ("tokens descending inside an expert", "permutation", permutation_tokens_descending,
     [(TL.test_handworked_layouts, ()), (TL.test_layout_bruteforce_random, (3,))]),
    ("inclusive expert offsets", "segment_offsets", offsets_inclusive,
     [(TL.test_handworked_layouts, ()), (TL.test_workload_layouts_structure, ())]),
    ("dedup counts pairs, not tokens", "dedup_counts", dedup_counts_pairs,
     [(TL.test_dedup_special_cases, ()), (TL.test_layout_bruteforce_random, (3,))]),
    ("bf16 rounding by truncation", "encode16", encode16_truncates,
     [(TW.test_encode16_matches_torch_rounding, ())]),
    ("stand-in scale off by one expert", "expert_standin", standin_expert_off_by_one,
     [(TW.test_standin_is_single_rounding_of_exact_product, (BF16, 8))]),
    ("combine drops slot 0's weight", "combine", combine_unit_weight_slot0,
     [(TW.test_combine_exact_closed_form, ())]),
    ("single-send rows token-major", "single_send_layout", single_send_token_major,
     [(TS.test_handworked_single_send_rows, ()), (TS.test_random_layouts, (0,))]),
    ("Gini without the 1/2", "gini", gini_doubled,
     [(TT.test_gini_closed_forms_and_textbook_formula, ())]),
    ("co-selection in both triangles", "coselection", coselection_both_triangles,
     [(TT.test_coselection_brute_force, ())]),
    ("locality as the off-diagonal share", "routing_stats", locality_off_diagonal,
     [(TT.test_locality_closed_form_uniform_over_eight_ranks, ()), (TT.test_hand_worked_two_ranks, ())]),
    ("larger shares on the last replicas", "replica_share_index", shares_larger_last,
     [(TE.test_share_index_against_expansion, ())]),
]


@pytest.mark.parametrize("what,name,wrong,pins", CASES, ids=[c[0] for c in CASES])
def test_planted_mistake_is_caught(monkeypatch, what, name, wrong, pins):
    for pin, args in pins:     # every pin passes on the oracle itself
        pin(*args)
    plant(monkeypatch, name, wrong)
    assert some_pin_fails(pins), f"no pin noticed: {what}"
