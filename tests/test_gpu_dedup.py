"""GPU parity for the per-group dedup variant: ep_get_group_layout, ep_dispatch
over a group layout, and ep_combine_groups, against the oracle.

Bar: the group layout (counts, offsets, rows, inverse map, flags) and the
receiver metadata are bit-exact, rows past the used ones are left untouched;
dispatch to the groups is bit-exact; the group combine is within
|gpu - ref| <= 8e-3 * max(|ref|, 1e-3) element-wise (fp32 against fp64 sums).
"""
import numpy as np
import pytest
import torch

import oracle
from combine_moe_layout_amd import binding as B
from combine_moe_layout_amd import workloads as W
from test_gpu_parity import assert_close_bf16, dev_bf16, host_bits, note, sample_tokens

pytestmark = pytest.mark.gpu

SENTINEL = -7


def gpu_group_layout(idx: np.ndarray, w, E: int, G: int, meta: bool = True):
    T, k = idx.shape
    gl = B.EpGroupLayout(T, k, E, G, with_recv_src=True)
    gl.recv_src.fill_(SENTINEL)
    R = gl.num_recv_rows
    ridx = torch.full((R, k), SENTINEL, dtype=torch.int64, device="cuda") if meta else None
    rw = torch.full((R, k), float(SENTINEL), dtype=torch.float32, device="cuda") if meta else None
    tw = torch.from_numpy(np.ascontiguousarray(w, np.float32)).cuda() if w is not None else None
    member = torch.full((T, G), 0x77, dtype=torch.uint8, device="cuda")
    B.ep_get_group_layout(torch.from_numpy(np.ascontiguousarray(idx, np.int64)).cuda(), tw, gl,
                          ridx, rw if w is not None else None, is_token_in_group=member)
    torch.cuda.synchronize()
    gl.is_token_in_group = member
    return gl, ridx, (rw if w is not None else None)


def compare_group_layout(idx, w, E, G, what, meta=True):
    o = oracle.group_layout(idx, w, E, G)
    gl, ridx, rw = gpu_group_layout(idx, w, E, G, meta)
    kg, used = o["kg"], o["rows_used"]
    eq = lambda a, b, key: np.testing.assert_array_equal(a, b, err_msg="%s: %s" % (what, key))
    eq(gl.num_tokens_per_expert.cpu().numpy(), o["num_tokens_per_group"], "group counts")
    eq(gl.num_tokens_per_group.cpu().numpy(), o["num_tokens_per_group"], "group counts (groups)")
    eq(gl.expert_offsets.cpu().numpy(), o["group_offsets"], "group offsets")
    eq(gl.slot_idx.cpu().numpy(), o["group_slot"], "group rows")
    src = np.full(gl.num_recv_rows, SENTINEL, np.int64)
    t_of, i_of = np.nonzero(o["group_slot"] >= 0)
    src[o["group_slot"][t_of, i_of]] = t_of * kg + i_of
    eq(gl.recv_src.cpu().numpy(), src, "recv_src (and untouched unused rows)")
    eq(gl.is_token_in_group.cpu().numpy(), o["is_token_in_group"], "is_token_in_group")
    assert int(gl.error_flags.cpu()[0]) == o["error_flags"], what
    if meta:
        gi = ridx.cpu().numpy()
        eq(gi[:used], o["recv_topk_idx"][:used], "recv_topk_idx")
        assert (gi[used:] == SENTINEL).all(), "%s: rows past the used ones were written" % what
        if rw is not None:
            gw = rw.cpu().numpy()
            eq(gw[:used].view(np.uint32), o["recv_topk_weights"][:used].view(np.uint32), "recv_topk_weights")
            assert (gw[used:] == SENTINEL).all()
    note("%s: T=%d k=%d E=%d G=%d kg=%d rows used %d of %d" % (
        what, idx.shape[0], idx.shape[1], E, G, kg, used, gl.num_recv_rows))
    return o, gl


# --------------------------------------------------------------------------- group layout
@pytest.mark.parametrize("name,G", [("dsv3", None), ("skewed", None), ("large", None),
                                     ("lowlat", None), ("tiny", 4), ("dsv3", 32), ("large", 64)])
def test_group_layout_named_workloads(name, G):
    wl = W.make(name)
    compare_group_layout(wl.topk_idx, wl.topk_weights, wl.E, G or wl.G, "%s G=%s" % (name, G or wl.G))


def _edge_cases():
    g = np.random.default_rng(21)
    cases = []
    # (T, k, E, G) shapes: one chunk and several, ragged tails, k above and below G,
    # k = 1, k = 64 (segments of a whole wave), G = 1, G = E
    for T, k, E, G in [(1, 8, 256, 8), (5, 3, 12, 4), (255, 8, 256, 8), (256, 8, 256, 8),
                       (257, 8, 256, 8), (2049, 1, 16, 16), (1000, 6, 64, 2), (700, 4, 64, 64),
                       (33, 64, 1024, 8), (40, 64, 64, 64), (3000, 5, 40, 1), (513, 7, 28, 7)]:
        idx = np.stack([g.permutation(E)[:k] if k <= E else g.integers(0, E, k)
                        for _ in range(T)]).astype(np.int64)
        cases.append(("T%d k%d E%d G%d" % (T, k, E, G), idx, E, G))
    # masks, bad ids and duplicates in one table
    T, k, E, G = 600, 8, 64, 8
    idx = g.integers(-1, E, size=(T, k)).astype(np.int64)
    idx[3] = -1                                  # a fully unrouted token
    idx[10, :] = 5                               # one expert eight times
    idx[20, 2] = E + 3                           # out of range: flag, skipped
    idx[30, 0] = -9                              # negative and not -1: flag
    cases.append(("masks+dups+bad", idx, E, G))
    # the same in one layout chunk (the one-launch layout, whose metadata
    # workgroup ORs in the table kernel's flag entries)
    small = idx[:100].copy()
    cases.append(("one chunk: masks+dups+bad", small, E, G))
    ok_small = np.where((small >= -1) & (small < E), small, -1)
    cases.append(("one chunk: masks+dups", ok_small, E, G))
    idx2 = np.full((50, 4), -1, np.int64)        # nothing routed at all
    cases.append(("all unrouted", idx2, 32, 4))
    idx3 = np.zeros((0, 8), np.int64)
    cases.append(("no tokens", idx3, 256, 8))
    return cases


@pytest.mark.parametrize("case", range(len(_edge_cases())))
def test_group_layout_edge_cases(case):
    what, idx, E, G = _edge_cases()[case]
    w = np.random.default_rng(case).random(idx.shape).astype(np.float32)
    compare_group_layout(idx, w, E, G, what)


def test_group_layout_without_metadata_or_weights():
    wl = W.make("dsv3", T=300)
    compare_group_layout(wl.topk_idx, None, wl.E, wl.G, "no weights", meta=True)
    compare_group_layout(wl.topk_idx, wl.topk_weights, wl.E, wl.G, "no metadata", meta=False)


def test_decode_group_layout_without_metadata_or_weights():
    """The one-launch form (at most 2048 pairs) with each optional output left
    out in turn, and with none of them: the slots and counts still match."""
    wl = W.make("dsv3", T=200)
    compare_group_layout(wl.topk_idx, None, wl.E, wl.G, "decode, no weights", meta=True)
    compare_group_layout(wl.topk_idx, wl.topk_weights, wl.E, wl.G, "decode, no metadata", meta=False)
    o = oracle.group_layout(wl.topk_idx, None, wl.E, wl.G)
    gl = B.EpGroupLayout(wl.T, wl.k, wl.E, wl.G)
    B.ep_get_group_layout(torch.from_numpy(wl.topk_idx).cuda(), None, gl)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(gl.slot_idx.cpu().numpy(), o["group_slot"])
    np.testing.assert_array_equal(gl.num_tokens_per_expert.cpu().numpy(), o["num_tokens_per_group"])


def test_group_layout_is_deterministic_and_repeatable():
    wl = W.make("skewed")
    a, _, _ = gpu_group_layout(wl.topk_idx, wl.topk_weights, wl.E, wl.G)
    first = a.slot_idx.cpu().numpy().copy()
    for _ in range(3):
        B.ep_get_group_layout(torch.from_numpy(wl.topk_idx).cuda(), None, a)
    torch.cuda.synchronize()
    assert (a.slot_idx.cpu().numpy() == first).all()


def test_second_level_layout_matches_the_expert_layout_at_full_size():
    """The receiving side's expert layout over the group rows gives the same
    per-expert counts, and inside each expert the same source tokens in the
    same order, as the expert layout over the original table (GPU only, at
    the benchmark's size)."""
    wl = W.make("dsv3")
    gl, ridx, _ = gpu_group_layout(wl.topk_idx, None, wl.E, wl.G)
    used = int(gl.expert_offsets[-1].item())
    first = B.EpLayout(wl.T, wl.k, wl.E, wl.G, with_recv_src=True)
    B.ep_get_layout(torch.from_numpy(wl.topk_idx).cuda(), first)
    second = B.EpLayout(used, wl.k, wl.E, wl.G, with_recv_src=True)
    B.ep_get_layout(ridx[:used].contiguous(), second)
    torch.cuda.synchronize()
    assert (first.num_tokens_per_expert.cpu() == second.num_tokens_per_expert.cpu()).all()
    n = int(first.expert_offsets[-1].item())
    kg = gl.num_topk
    row_token = (gl.recv_src.cpu().numpy()[:used] // kg).astype(np.int64)
    src1 = first.recv_src.cpu().numpy()[:n] // wl.k
    src2 = row_token[second.recv_src.cpu().numpy()[:n] // wl.k]
    assert (src1 == src2).all()


# --------------------------------------------------------------------------- dispatch to the groups
@pytest.mark.parametrize("name,T,dtype", [("dsv3", 256, B.EP_FP8_E4M3), ("dsv3", 256, B.EP_FP8_E4M3_POW2),
                                           ("skewed", 300, B.EP_BF16), ("large", 512, B.EP_FP8_E4M3),
                                           ("lowlat", None, B.EP_FP8_E4M3), ("tiny", None, B.EP_BF16)])
def test_dispatch_to_groups(name, T, dtype):
    wl = W.make(name, T=T)
    G = wl.G if name != "tiny" else 4
    o = oracle.group_layout(wl.topk_idx, None, wl.E, G)
    gl, _, _ = gpu_group_layout(wl.topk_idx, None, wl.E, G, meta=False)
    R, used, H = gl.num_recv_rows, o["rows_used"], wl.H
    x = dev_bf16(wl.x_bits)
    note("dispatch to groups %s T=%d H=%d dtype=%d rows %d" % (name, wl.T, H, dtype, used))
    if dtype == B.EP_BF16:
        recv = torch.empty((R, H), dtype=torch.bfloat16, device="cuda")
        recv.view(torch.int16).fill_(0x1357)
        B.ep_dispatch(x, gl, dtype, recv)
        got = host_bits(recv)
        want = oracle.dispatch_bf16(wl.x_bits, o["group_slot"], R)
        assert (got[:used] == want[:used]).all() and (got[used:] == 0x1357).all()
    else:
        q = torch.full((R, H), 0x5A, dtype=torch.uint8, device="cuda")
        s = torch.full((R, H // 128), 3.0, dtype=torch.float32, device="cuda")
        B.ep_dispatch(x, gl, dtype, q, s)
        fn = oracle.dispatch_fp8 if dtype == B.EP_FP8_E4M3 else oracle.dispatch_fp8_pow2
        oq, os_ = fn(wl.x_bits, o["group_slot"], R)
        gq, gs = q.cpu().numpy(), s.cpu().numpy()
        assert (gq[:used] == oq[:used]).all(), "codes differ"
        assert (gs[:used].view(np.uint32) == os_[:used].view(np.uint32)).all(), "scales differ"
        assert (gq[used:] == 0x5A).all() and (gs[used:] == 3.0).all()


def test_dispatch_to_groups_full_size_sampled():
    wl = W.make("dsv3")
    o = oracle.group_layout(wl.topk_idx, None, wl.E, wl.G)
    gl, _, _ = gpu_group_layout(wl.topk_idx, None, wl.E, wl.G, meta=False)
    R = gl.num_recv_rows
    q = torch.empty((R, wl.H), dtype=torch.uint8, device="cuda")
    s = torch.empty((R, wl.H // 128), dtype=torch.float32, device="cuda")
    B.ep_dispatch(dev_bf16(wl.x_bits), gl, B.EP_FP8_E4M3, q, s)
    torch.cuda.synchronize()
    note("dispatch to groups, full size: %d rows instead of %d" % (o["rows_used"], wl.T * wl.k))
    qh, sh = q.cpu().numpy(), s.cpu().numpy()
    for t in sample_tokens(wl.T, 48):
        rows = o["group_slot"][t][o["group_slot"][t] >= 0]
        oq, os_ = oracle.quantize_token_fp8(wl.x_bits[t])
        assert (qh[rows] == oq).all(), "token %d codes" % t
        assert (sh[rows].view(np.uint32) == os_.view(np.uint32)).all(), "token %d scales" % t


# --------------------------------------------------------------------------- group combine
@pytest.mark.parametrize("name,T,H,G", [("tiny", None, None, 4), ("dsv3", 256, None, None),
                                         ("lowlat", None, None, None), ("large", 512, None, None),
                                         ("dsv3", 40, 24, None), ("dsv3", 9, 16512, None),
                                         ("large", 300, 4096, 64), ("skewed", 100, 7168, 1),
                                         # prefill-sized, packed 1024-lane workgroups, ragged tail
                                         ("large", 1001, 4096, None), ("dsv3", 1027, 2048, 8)])
def test_combine_groups_random_rows(name, T, H, G):
    wl = W.make(name, T=T, H=H)
    G = G or wl.G
    o = oracle.group_layout(wl.topk_idx, None, wl.E, G)
    gl, _, _ = gpu_group_layout(wl.topk_idx, None, wl.E, G, meta=False)
    z = W.random_expert_outputs(gl.num_recv_rows, wl.H, seed=31)
    out = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda")
    B.ep_combine_groups(dev_bf16(z), gl, out)
    torch.cuda.synchronize()
    assert_close_bf16(host_bits(out), oracle.combine_groups(z, o["group_slot"]),
                      "group combine %s T=%d H=%d G=%d" % (name, wl.T, wl.H, G))


def test_combine_groups_full_size_sampled():
    wl = W.make("dsv3")
    o = oracle.group_layout(wl.topk_idx, None, wl.E, wl.G)
    gl, _, _ = gpu_group_layout(wl.topk_idx, None, wl.E, wl.G, meta=False)
    z = W.random_expert_outputs(gl.num_recv_rows, wl.H, seed=32)
    out = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda")
    B.ep_combine_groups(dev_bf16(z), gl, out)
    torch.cuda.synchronize()
    toks = sample_tokens(wl.T, 64)
    assert_close_bf16(host_bits(out)[toks], oracle.combine_groups_tokens(z, o["group_slot"], toks),
                      "group combine full size (sampled)")


def test_dedup_path_with_identity_experts():
    """Group layout and dispatch on the GPU, the receiving side's weighted sum
    (identity experts) from the oracle, group combine on the GPU; against the
    oracle's path end to end."""
    wl = W.make("dsv3", T=192, H=1024)
    o = oracle.group_layout(wl.topk_idx, wl.topk_weights, wl.E, wl.G)
    gl, ridx, rw = gpu_group_layout(wl.topk_idx, wl.topk_weights, wl.E, wl.G)
    used, R, k = o["rows_used"], gl.num_recv_rows, wl.k
    recv = torch.zeros((R, wl.H), dtype=torch.bfloat16, device="cuda")
    B.ep_dispatch(dev_bf16(wl.x_bits), gl, B.EP_BF16, recv)
    got_recv = host_bits(recv)[:used]
    self_slot = np.repeat(np.arange(used, dtype=np.int32)[:, None], k, axis=1)
    z = np.zeros((R, wl.H), np.uint16)
    z[:used] = oracle.combine(got_recv, rw.cpu().numpy()[:used], self_slot)
    out = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda")
    B.ep_combine_groups(dev_bf16(z), gl, out)
    torch.cuda.synchronize()
    o_recv = oracle.dispatch_bf16(wl.x_bits, o["group_slot"], R)[:used]
    o_z = oracle.combine(o_recv, o["recv_topk_weights"][:used], self_slot)
    ref = oracle.combine_groups(o_z, o["group_slot"])
    assert_close_bf16(host_bits(out), ref, "dedup path, identity experts")
