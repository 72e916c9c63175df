"""Pins for the oracle's routing layout (CPU only).

Checked against hand-worked fixtures, library routines that compute the same
quantities another way (numpy bincount, cumsum, stable argsort), a pure-Python
brute force on tiny inputs, and invariants on every named workload.
"""
import json
import os

import numpy as np
import pytest

import oracle
from combine_moe_layout_amd import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_layout_golden():
    with open(os.path.join(GOLDEN, "layout_tiny.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        out = oracle.layout(np.array(c["topk_idx"], np.int64), c["E"], c["G"], c["cap"])
        why = c["why"]
        assert out["num_tokens_per_expert"].tolist() == c["num_tokens_per_expert"], why
        assert out["expert_offsets"].tolist() == c["expert_offsets"], why
        assert out["num_tokens_per_group"].tolist() == c["num_tokens_per_group"], why
        assert out["slot_idx"].tolist() == c["slot_idx"], why
        assert out["recv_src"].tolist() == c["recv_src"], why
        assert out["error_flags"] == c["error_flags"], why


def _brute(topk_idx, E, G, cap):
    """Definition by counting, O(P^2): rank of pair p inside its expert is the
    number of earlier pairs with the same expert."""
    flat = [int(v) for v in np.asarray(topk_idx).reshape(-1)]
    valid = [0 <= e < E for e in flat]
    counts = [sum(1 for e, v in zip(flat, valid) if v and e == x) for x in range(E)]
    offs = [cap * x for x in range(E + 1)] if cap else [sum(counts[:x]) for x in range(E + 1)]
    flags = 1 if any((not v) and e != -1 for e, v in zip(flat, valid)) else 0
    slots = []
    for p, e in enumerate(flat):
        if not valid[p]:
            slots.append(-1)
            continue
        r = sum(1 for q in range(p) if valid[q] and flat[q] == e)
        if cap and r >= cap:
            slots.append(-1)
            flags |= 2
        else:
            slots.append(offs[e] + r)
    per = E // G
    groups = [sum(counts[g * per:(g + 1) * per]) for g in range(G)]
    return counts, offs, groups, slots, flags


@pytest.mark.parametrize("seed", range(40))
def test_layout_brute_force_tiny(seed):
    g = np.random.default_rng(seed)
    T = int(g.integers(1, 17))
    k = int(g.integers(1, 5))
    G = int(g.choice([1, 2, 4]))
    E = G * int(g.integers(1, 5))
    cap = int(g.choice([0, 0, 1, 2, 3]))
    # ids in [-2, E+1]: unrouted (-1), bad ids (-2, E, E+1), duplicates in a row
    idx = g.integers(-2, E + 2, size=(T, k)).astype(np.int64)
    mostly_valid = g.random((T, k)) < 0.6
    idx = np.where(mostly_valid, g.integers(0, E, size=(T, k)), idx).astype(np.int64)
    counts, offs, groups, slots, flags = _brute(idx, E, G, cap)
    out = oracle.layout(idx, E, G, cap)
    assert out["num_tokens_per_expert"].tolist() == counts
    assert out["expert_offsets"].tolist() == offs
    assert out["num_tokens_per_group"].tolist() == groups
    assert out["slot_idx"].reshape(-1).tolist() == slots
    assert out["error_flags"] == flags


def _check_against_library(idx, E, G, cap):
    out = oracle.layout(idx, E, G, cap)
    flat = idx.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    cnt = np.bincount(flat[valid], minlength=E)
    assert (out["num_tokens_per_expert"] == cnt).all()
    if cap == 0:
        assert (out["expert_offsets"] == np.concatenate([[0], np.cumsum(cnt)])).all()
    else:
        assert (out["expert_offsets"] == cap * np.arange(E + 1)).all()
    assert (out["num_tokens_per_group"] == cnt.reshape(G, -1).sum(1)).all()
    # slots: position in the stable sort of the valid pairs by expert
    order = np.argsort(np.where(valid, flat, E), kind="stable")[: valid.sum()]
    rank_in_expert = np.empty(flat.size, np.int64)
    sorted_e = flat[order]
    first = np.searchsorted(sorted_e, sorted_e, side="left")
    rank_in_expert[order] = np.arange(order.size) - first
    slot = out["slot_idx"].reshape(-1)
    kept = valid & ((rank_in_expert < cap) if cap else True)
    expect = np.where(kept, out["expert_offsets"][np.where(valid, flat, 0)] + rank_in_expert, -1)
    assert (slot == expect).all()
    # bijection onto the used rows; recv_src inverts slot
    used = slot[slot >= 0]
    assert np.unique(used).size == used.size
    if cap == 0:
        assert (np.sort(used) == np.arange(valid.sum())).all()
    src = out["recv_src"]
    assert (src[used] == np.nonzero(slot >= 0)[0]).all()
    flags = (1 if ((~valid) & (flat != -1)).any() else 0) | (2 if cap and (cnt > cap).any() else 0)
    assert out["error_flags"] == flags
    return out


@pytest.mark.parametrize("name", list(workloads.CONFIGS))
def test_layout_named_workloads_vs_library(name):
    T0, H0, E, G, k, cap, fp8, kind = workloads.CONFIGS[name]
    idx, w = workloads.route(kind, T0, E, k, G, seed=0)
    out = _check_against_library(idx, E, G, cap)
    # no masks in the generators: every pair is counted
    assert out["num_tokens_per_expert"].sum() == T0 * k


def test_layout_random_with_masks_and_overflow():
    g = np.random.default_rng(3)
    for cap in (0, 5, 40):
        idx = g.integers(-1, 33, size=(500, 6)).astype(np.int64)
        idx[idx == 32] = 77  # bad id
        _check_against_library(idx, 32, 4, cap)


def test_layout_empty_and_degenerate():
    out = oracle.layout(np.zeros((0, 4), np.int64), 8, 2, 0)
    assert out["num_tokens_per_expert"].sum() == 0 and out["expert_offsets"].tolist() == [0] * 9
    # every pair to one expert
    idx = np.full((64, 4), 5, np.int64)
    out = _check_against_library(idx, 8, 2, 0)
    assert out["slot_idx"].reshape(-1).tolist() == list(range(256))
    # all unrouted
    out = oracle.layout(np.full((10, 3), -1, np.int64), 4, 1, 0)
    assert (out["slot_idx"] == -1).all() and out["error_flags"] == 0
    with pytest.raises(ValueError):
        oracle.layout(np.zeros((2, 2), np.int64), 6, 4, 0)  # E % G != 0
