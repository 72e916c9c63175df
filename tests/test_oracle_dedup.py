"""Pins for the oracle's per-group dedup variant (CPU only).

The variant sends a token once to every group holding one of its experts
(rows group-major, ascending token inside a group), with the token's top-k
list masked to that group, and sums the returned group rows per token.  The
oracle is checked against hand-worked fixtures, a pure-Python definition on
tiny inputs, a numpy stable sort, the expert layout (which is pinned on its
own) in the cases where the two must agree, and conservation invariants.
"""
import json
import os

import numpy as np
import pytest

import oracle
from combine_moe_layout_amd import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden():
    with open(os.path.join(GOLDEN, "group_layout_tiny.json")) as f:
        return json.load(f)


def test_group_layout_golden():
    for c in _golden()["cases"]:
        out = oracle.group_layout(np.array(c["topk_idx"], np.int64),
                                  np.array(c["topk_weights"], np.float32), c["E"], c["G"])
        why = c["why"]
        used = out["rows_used"]
        assert out["group_idx"].tolist() == c["group_idx"], why
        assert out["num_tokens_per_group"].tolist() == c["num_tokens_per_group"], why
        assert out["group_offsets"].tolist() == c["group_offsets"], why
        assert out["group_slot"].tolist() == c["group_slot"], why
        assert out["recv_token"][:used].tolist() == c["recv_token"], why
        assert out["recv_topk_idx"][:used].tolist() == c["recv_topk_idx"], why
        assert out["recv_topk_weights"][:used].tolist() == c["recv_topk_weights"], why
        assert out["error_flags"] == c["error_flags"], why
        # rows past the used ones are left as the caller set them
        assert (out["recv_token"][used:] == -1).all() and (out["recv_topk_idx"][used:] == -1).all()


def test_combine_groups_golden():
    c = _golden()["combine_groups"]
    out = oracle.combine_groups(np.array(c["z"], np.uint16), np.array(c["group_slot"], np.int32))
    assert out.tolist() == c["out"], c["why"]


def _brute(topk_idx, w, E, G):
    """The definition by counting, in plain Python."""
    T, k = topk_idx.shape
    per = E // G
    kg = min(k, G)
    flags = 0
    groups = []
    for t in range(T):
        s = set()
        for j in range(k):
            e = int(topk_idx[t, j])
            if e == -1:
                continue
            if not 0 <= e < E:
                flags |= 1
                continue
            s.add(e // per)
        groups.append(sorted(s))
    counts = [sum(1 for t in range(T) if g in groups[t]) for g in range(G)]
    offs = [sum(counts[:g]) for g in range(G + 1)]
    gidx = [groups[t] + [-1] * (kg - len(groups[t])) for t in range(T)]
    slot, tok, ridx, rw = [], {}, {}, {}
    for t in range(T):
        row_list = []
        for g in gidx[t]:
            if g < 0:
                row_list.append(-1)
                continue
            r = offs[g] + sum(1 for u in range(t) if g in groups[u])
            row_list.append(r)
            tok[r] = t
            ridx[r] = [int(e) if 0 <= e < E and e // per == g else -1 for e in topk_idx[t]]
            rw[r] = [float(w[t, j]) if 0 <= topk_idx[t, j] < E and topk_idx[t, j] // per == g else 0.0
                     for j in range(k)]
        slot.append(row_list)
    return gidx, counts, offs, slot, tok, ridx, rw, flags


@pytest.mark.parametrize("seed", range(40))
def test_group_layout_brute_force_tiny(seed):
    g = np.random.default_rng(seed)
    G = int(g.choice([1, 2, 3, 4, 8]))
    E = G * int(g.integers(1, 4))
    T = int(g.integers(0, 14))
    k = int(g.integers(1, 7))
    idx = g.integers(-1, E, size=(T, k)).astype(np.int64)   # -1 and duplicates occur
    if T and seed % 3 == 0:
        idx[g.integers(0, T), g.integers(0, k)] = E + int(g.integers(0, 5))  # a bad id
    w = g.random((T, k)).astype(np.float32)
    out = oracle.group_layout(idx, w, E, G)
    gidx, counts, offs, slot, tok, ridx, rw, flags = _brute(idx, w, E, G)
    assert out["group_idx"].tolist() == (gidx if T else [])
    assert out["num_tokens_per_group"].tolist() == counts
    assert out["group_offsets"].tolist() == offs
    assert out["group_slot"].tolist() == (slot if T else [])
    assert out["error_flags"] == flags
    member = [[1 if gg in gidx[t] else 0 for gg in range(G)] for t in range(T)]
    assert out["is_token_in_group"].tolist() == member
    for r in range(out["rows_used"]):
        assert out["recv_token"][r] == tok[r]
        assert out["recv_topk_idx"][r].tolist() == ridx[r]
        assert out["recv_topk_weights"][r].tolist() == pytest.approx(rw[r], abs=0)


def _entries(topk_idx, E, G):
    """(token, group) presence by numpy indexing."""
    T, k = topk_idx.shape
    valid = (topk_idx >= 0) & (topk_idx < E)
    present = np.zeros((T, G), bool)
    rows = np.broadcast_to(np.arange(T)[:, None], (T, k))[valid]
    present[rows, topk_idx[valid] // (E // G)] = True
    return present


@pytest.mark.parametrize("name", ["dsv3", "skewed", "large", "lowlat"])
def test_group_layout_matches_a_stable_sort(name):
    wl = workloads.make(name, seed=3)
    out = oracle.group_layout(wl.topk_idx, wl.topk_weights, wl.E, wl.G)
    present = _entries(wl.topk_idx, wl.E, wl.G)
    t_of, g_of = np.nonzero(present)              # token-major, groups ascending per token
    assert (out["num_tokens_per_group"] == present.sum(0)).all()
    assert (out["is_token_in_group"] == present).all()
    assert (out["group_offsets"] == np.concatenate([[0], np.cumsum(present.sum(0))])).all()
    order = np.argsort(g_of, kind="stable")       # group-major, token order kept
    rows = np.empty_like(order)
    rows[order] = np.arange(order.size)
    kg = out["kg"]
    want = np.full((wl.T, kg), -1, np.int64)
    pos = np.concatenate([np.arange(c) for c in present.sum(1)])
    want[t_of, pos] = rows
    assert (out["group_slot"] == want).all()
    want_gidx = np.full((wl.T, kg), -1, np.int64)
    want_gidx[t_of, pos] = g_of
    assert (out["group_idx"] == want_gidx).all()
    assert (out["recv_token"][:order.size] == t_of[order]).all()


@pytest.mark.parametrize("name", ["dsv3", "skewed", "lowlat"])
def test_second_level_layout_is_the_expert_layout(name):
    """The receiving side lays out its rows by expert; with rows ascending in
    token inside each group, that must give the expert layout's counts and,
    inside every expert, the same source tokens in the same order."""
    wl = workloads.make(name, seed=4)
    g = oracle.group_layout(wl.topk_idx, wl.topk_weights, wl.E, wl.G)
    used = g["rows_used"]
    first = oracle.layout(wl.topk_idx, wl.E, wl.G, 0)
    second = oracle.layout(g["recv_topk_idx"][:used], wl.E, wl.G, 0)
    assert (second["num_tokens_per_expert"] == first["num_tokens_per_expert"]).all()
    n = int(first["expert_offsets"][-1])
    src1 = first["recv_src"][:n] // wl.k                      # source token of each expert row
    src2 = g["recv_token"][second["recv_src"][:n] // wl.k]    # via the group row
    assert (src1 == src2).all()


@pytest.mark.parametrize("name", ["dsv3", "large"])
def test_receiver_metadata_partitions_each_token(name):
    wl = workloads.make(name, seed=5)
    g = oracle.group_layout(wl.topk_idx, wl.topk_weights, wl.E, wl.G)
    used = g["rows_used"]
    tok = g["recv_token"][:used]
    ridx, rw = g["recv_topk_idx"][:used], g["recv_topk_weights"][:used]
    # every valid (t, j) appears in exactly one of t's rows, with its weight
    hits = np.zeros(wl.topk_idx.shape, np.int64)
    np.add.at(hits, tok, (ridx >= 0).astype(np.int64))
    valid = (wl.topk_idx >= 0) & (wl.topk_idx < wl.E)
    assert (hits == valid).all()
    wsum = np.zeros(wl.topk_idx.shape, np.float64)
    np.add.at(wsum, tok, rw.astype(np.float64))
    assert (wsum == np.where(valid, wl.topk_weights, 0)).all()
    # a row's kept experts all belong to its group, and the group is the row's
    grp_of_row = np.searchsorted(g["group_offsets"], np.arange(used), side="right") - 1
    kept = ridx >= 0
    assert (ridx[kept] // (wl.E // wl.G) == np.broadcast_to(grp_of_row[:, None], ridx.shape)[kept]).all()
    assert kept.any(axis=1).all()


def test_one_group_and_one_group_per_expert():
    rng = np.random.default_rng(9)
    T, k, E = 64, 4, 16
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int64)
    idx[::7, 1] = -1
    w = rng.random((T, k)).astype(np.float32)
    # G = 1: one row per token, in token order, carrying the token's whole list
    g1 = oracle.group_layout(idx, w, E, 1)
    assert g1["group_slot"][:, 0].tolist() == list(range(T))
    assert (g1["recv_topk_idx"][:T] == idx).all()
    # G = E with distinct experts: the dedup layout is the expert layout
    gE = oracle.group_layout(idx, w, E, E)
    lay = oracle.layout(idx, E, E, 0)
    for t in range(T):
        valid = idx[t] >= 0
        order = np.argsort(idx[t][valid])
        assert gE["group_slot"][t][:valid.sum()].tolist() == lay["slot_idx"][t][valid][order].tolist()
    assert (gE["num_tokens_per_group"] == lay["num_tokens_per_expert"]).all()


def test_combine_groups_is_the_unit_weight_combine():
    """With unit weights the group combine is the ordinary combine over the
    group rows (the ordinary combine is pinned on its own)."""
    rng = np.random.default_rng(11)
    wl = workloads.make("tiny", seed=2)
    g = oracle.group_layout(wl.topk_idx, wl.topk_weights, 8, 4)
    used = g["rows_used"]
    z = workloads.random_expert_outputs(used, wl.H, seed=7)
    ones = np.ones(g["group_slot"].shape, np.float32)
    assert (oracle.combine_groups(z, g["group_slot"]) == oracle.combine(z, ones, g["group_slot"])).all()
    toks = rng.choice(wl.T, 9, replace=False)
    assert (oracle.combine_groups_tokens(z, g["group_slot"], toks)
            == oracle.combine_groups(z, g["group_slot"])[toks]).all()


def _expert_side(recv_bits, rw):
    """What the receiving side returns under identity experts: each row's
    weighted sum over its kept experts, rounded to bf16 (the ordinary combine,
    every entry reading the row itself)."""
    used, k = rw.shape
    self_slot = np.repeat(np.arange(used, dtype=np.int32)[:, None], k, axis=1)
    return oracle.combine(recv_bits, rw, self_slot)


@pytest.mark.parametrize("name", ["tiny", "dsv3"])
def test_dedup_round_trip(name):
    wl = workloads.make(name, seed=6, T=64 if name == "dsv3" else None)
    E, G = wl.E, (4 if name == "tiny" else wl.G)
    g = oracle.group_layout(wl.topk_idx, wl.topk_weights, E, G)
    used = g["rows_used"]
    recv = oracle.dispatch_bf16(wl.x_bits, g["group_slot"], used)
    assert (recv == wl.x_bits[g["recv_token"][:used]]).all()           # one copy per (t, g)
    z = _expert_side(recv, g["recv_topk_weights"][:used])
    out = oracle.combine_groups(z, g["group_slot"])
    x = workloads.bf16_bits_to_float32(wl.x_bits).astype(np.float64)
    got = workloads.bf16_bits_to_float32(out).astype(np.float64)
    # weights sum to 1 per token: two bf16 roundings away from x at most
    assert (np.abs(got - x) <= 2 * 2.0 ** -8 * np.abs(x) + 1e-30).all()
    # with one group there is only one row per token, and the trip is exact
    g1 = oracle.group_layout(wl.topk_idx, wl.topk_weights, E, 1)
    recv1 = oracle.dispatch_bf16(wl.x_bits, g1["group_slot"], g1["rows_used"])
    out1 = oracle.combine_groups(_expert_side(recv1, g1["recv_topk_weights"][:g1["rows_used"]]),
                                 g1["group_slot"])
    assert ((out1 & 0x7FFF) == (wl.x_bits & 0x7FFF)).all()


def test_group_layout_rejects_bad_shapes():
    idx = np.zeros((2, 2), np.int64)
    with pytest.raises(ValueError):
        oracle.group_layout(idx, None, 6, 4)     # E % G != 0
    empty = oracle.group_layout(np.zeros((0, 3), np.int64), None, 8, 2)
    assert empty["rows_used"] == 0 and empty["group_offsets"].tolist() == [0, 0, 0]
