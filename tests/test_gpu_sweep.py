"""GPU parity over seeded random configurations: layout, dispatch (bf16, FP8,
power-of-two FP8, MXFP8) and combine against the oracle, on shapes the named
workloads do not reach (odd token counts and top-k, many or few experts and
groups, small capacities with drops, masked entries, narrow and wide rows);
the one-launch decode path (ep_layout_dispatch at most 4096 pairs, top-k at
most 8) and the per-group dedup path over random configurations of their own.

Same bar as the other parity tests: layout and dispatch bit-exact, combine
within |gpu - ref| <= 8e-3 * max(|ref|, 1e-3).
"""
import numpy as np
import pytest
import torch

import oracle
from combine_moe_layout_amd import binding as B
from combine_moe_layout_amd import workloads as W
from test_gpu_dedup import compare_group_layout
from test_gpu_parity import (assert_close_bf16, assert_layout_equal, dev_bf16, gpu_layout, host_bits,
                             layout_to_host, note)

pytestmark = pytest.mark.gpu

DTYPES = [B.EP_BF16, B.EP_FP8_E4M3, B.EP_FP8_E4M3_POW2, B.EP_MXFP8_E4M3]


def _config(seed):
    g = np.random.default_rng(1000 + seed)
    k = int(g.integers(1, 11))
    G = int(g.choice([1, 2, 4, 8, 16]))
    E = G * int(g.integers(max(1, -(-k // G)), 65))          # at least k experts
    dtype = DTYPES[seed % len(DTYPES)]
    fp8 = dtype != B.EP_BF16
    H = 128 * int(g.integers(1, 24)) if fp8 else 8 * int(g.integers(1, 400))
    T = int(g.integers(1, max(2, 2_000_000 // (H * k))))
    T = min(T, 3000)
    cap = int(g.integers(1, 64)) if seed % 3 == 0 else 0
    return T, H, E, G, k, cap, dtype


@pytest.mark.parametrize("seed", range(96))
def test_random_configuration(seed):
    T, H, E, G, k, cap, dtype = _config(seed)
    note("sweep seed %d: T=%d H=%d E=%d G=%d k=%d cap=%d dtype=%d" % (seed, T, H, E, G, k, cap, dtype))
    wl = W.custom(T, H, E, k, G=G, cap=cap, fp8=dtype != B.EP_BF16, seed=seed)
    idx = wl.topk_idx.copy()
    g = np.random.default_rng(seed)
    idx[g.random(idx.shape) < 0.05] = -1                     # masked entries
    ol = oracle.layout(idx, E, G, cap)
    lay = gpu_layout(idx, E, G, cap)
    assert_layout_equal(layout_to_host(lay), ol, "sweep %d layout" % seed)

    R = lay.num_recv_rows
    x = dev_bf16(wl.x_bits)
    used = np.zeros(R, bool)
    used[ol["slot_idx"][ol["slot_idx"] >= 0]] = True
    if dtype == B.EP_BF16:
        recv = torch.zeros((R, H), dtype=torch.bfloat16, device="cuda")
        B.ep_dispatch(x, lay, dtype, recv)
        got = host_bits(recv)
        assert (got[used] == oracle.dispatch_bf16(wl.x_bits, ol["slot_idx"], R)[used]).all()
        y_bits = W.random_expert_outputs(R, H, seed=seed)
    else:
        mx = dtype == B.EP_MXFP8_E4M3
        q = torch.zeros((R, H), dtype=torch.uint8, device="cuda")
        s = (torch.zeros((R, H // 32), dtype=torch.uint8, device="cuda") if mx else
             torch.zeros((R, H // 128), dtype=torch.float32, device="cuda"))
        B.ep_dispatch(x, lay, dtype, q, s)
        fn = (oracle.dispatch_mxfp8 if mx else
              oracle.dispatch_fp8_pow2 if dtype == B.EP_FP8_E4M3_POW2 else oracle.dispatch_fp8)
        oq, os_ = fn(wl.x_bits, ol["slot_idx"], R)
        qh, sh = q.cpu().numpy(), s.cpu().numpy()
        assert (qh[used] == oq[used]).all(), "codes"
        if mx:
            assert (sh[used] == os_[used]).all(), "E8M0 bytes"
        else:
            assert (sh[used].view(np.uint32) == os_[used].view(np.uint32)).all(), "scales"
        y_bits = oracle.dequant_mxfp8(oq, os_) if mx else oracle.dequant_fp8(oq, os_)
        # the combine of FP8 expert outputs, both sides on the oracle's
        # dispatched codes and scales (a token's rows are copies of it and the
        # weights are positive, so no sum cancels)
        out8 = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
        w = torch.from_numpy(wl.topk_weights).cuda()
        q8, s8 = torch.from_numpy(oq).cuda(), torch.from_numpy(os_).cuda()
        if mx:
            B.ep_combine_mxfp8(q8, s8, w, lay, out8)
            ref8 = oracle.combine_mxfp8(oq, os_, wl.topk_weights, ol["slot_idx"])
        else:
            B.ep_combine_fp8(q8, s8, w, lay, out8)
            ref8 = oracle.combine_fp8(oq, os_, wl.topk_weights, ol["slot_idx"])
        torch.cuda.synchronize()
        assert_close_bf16(host_bits(out8), ref8, "sweep %d FP8 combine" % seed)

    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    B.ep_combine(dev_bf16(y_bits), torch.from_numpy(wl.topk_weights).cuda(), lay, out)
    torch.cuda.synchronize()
    assert_close_bf16(host_bits(out), oracle.combine(y_bits, wl.topk_weights, ol["slot_idx"]),
                      "sweep %d combine" % seed)


def _fused_config(seed):
    g = np.random.default_rng(5000 + seed)
    k = int(g.integers(1, 9))
    G = int(g.choice([1, 2, 4, 8]))
    E = G * int(g.integers(max(1, -(-k // G)), 129 // G + 1))
    T = int(g.integers(1, 4096 // k + 1))
    dtype = DTYPES[seed % len(DTYPES)]
    H = 128 * int(g.integers(1, 72)) if dtype != B.EP_BF16 else 8 * int(g.integers(1, 1100))
    cap = int(g.integers(1, 2 * max(1, T * k // E) + 2)) if seed % 2 == 0 else 0
    return T, H, E, G, k, cap, dtype


@pytest.mark.parametrize("seed", range(64))
def test_random_fused_configuration(seed):
    """ep_layout_dispatch on decode-sized batches: the one-launch kernel,
    against the oracle's layout and dispatch (rows past one pass of the lanes
    loop; padded layouts drop)."""
    T, H, E, G, k, cap, dtype = _fused_config(seed)
    note("fused sweep seed %d: T=%d H=%d E=%d G=%d k=%d cap=%d dtype=%d" % (seed, T, H, E, G, k, cap, dtype))
    wl = W.custom(T, H, E, k, G=G, cap=cap, fp8=dtype != B.EP_BF16, seed=seed)
    idx = wl.topk_idx.copy()
    idx[np.random.default_rng(seed).random(idx.shape) < 0.05] = -1
    ol = oracle.layout(idx, E, G, cap)
    lay = B.EpLayout(T, k, E, G, cap, with_recv_src=True)
    lay.recv_src.fill_(-1)
    R = lay.num_recv_rows
    x = dev_bf16(wl.x_bits)
    fp8 = dtype != B.EP_BF16
    q = torch.full((R, H), 0x5A, dtype=torch.uint8 if fp8 else torch.int16, device="cuda")
    s = None
    if fp8:
        s = (torch.full((R, H // 32), 0xA5, dtype=torch.uint8, device="cuda") if dtype == B.EP_MXFP8_E4M3
             else torch.full((R, H // 128), -3.0, dtype=torch.float32, device="cuda"))
    B.ep_layout_dispatch(torch.from_numpy(idx).cuda(), lay, x, dtype,
                         q if fp8 else q.view(torch.bfloat16), s)
    assert_layout_equal(layout_to_host(lay), ol, "fused sweep %d layout" % seed)
    used = np.zeros(R, bool)
    used[ol["slot_idx"][ol["slot_idx"] >= 0]] = True
    qh = q.cpu().numpy()
    if fp8:
        fn = (oracle.dispatch_mxfp8 if dtype == B.EP_MXFP8_E4M3 else
              oracle.dispatch_fp8_pow2 if dtype == B.EP_FP8_E4M3_POW2 else oracle.dispatch_fp8)
        oq, os_ = fn(wl.x_bits, ol["slot_idx"], R)
        sh = s.cpu().numpy()
        assert (qh[used] == oq[used]).all() and (qh[~used] == 0x5A).all(), "codes"
        assert (sh[used].view(np.uint8) == np.ascontiguousarray(os_[used]).view(np.uint8)).all(), "scales"
    else:
        orecv = oracle.dispatch_bf16(wl.x_bits, ol["slot_idx"], R)
        assert (qh.view(np.uint16)[used] == orecv[used]).all() and (qh[~used] == 0x5A).all(), "rows"


def _group_config(seed):
    g = np.random.default_rng(7000 + seed)
    k = int(g.integers(1, 17))
    G = int(g.choice([1, 2, 3, 4, 8, 16, 32]))
    E = G * int(g.integers(max(1, -(-k // G)), 33))
    T = int(g.integers(1, 3000))
    H = 8 * int(g.integers(1, 300))
    return T, H, E, G, k


@pytest.mark.parametrize("seed", range(24))
def test_random_group_configuration(seed):
    """The per-group dedup path on random shapes: group layout, receiver
    metadata, bf16 dispatch to the groups and the group combine against the
    oracle."""
    T, H, E, G, k = _group_config(seed)
    note("group sweep seed %d: T=%d H=%d E=%d G=%d k=%d" % (seed, T, H, E, G, k))
    wl = W.custom(T, H, E, k, G=G, seed=seed)
    idx = wl.topk_idx.copy()
    idx[np.random.default_rng(seed).random(idx.shape) < 0.05] = -1
    o, gl = compare_group_layout(idx, wl.topk_weights, E, G, "group sweep %d" % seed)
    Rg = gl.num_recv_rows
    z_rows = torch.full((Rg, H), 0x1234, dtype=torch.int16, device="cuda")
    B.ep_dispatch(dev_bf16(wl.x_bits), gl, B.EP_BF16, z_rows.view(torch.bfloat16))
    zh = z_rows.cpu().numpy().view(np.uint16)
    used = o["rows_used"]
    assert (zh[:used] == oracle.dispatch_bf16(wl.x_bits, o["group_slot"], Rg)[:used]).all()
    assert (zh[used:] == 0x1234).all()
    zz = W.random_expert_outputs(Rg, H, seed=seed)
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    B.ep_combine_groups(dev_bf16(zz), gl, out)
    torch.cuda.synchronize()
    assert_close_bf16(host_bits(out), oracle.combine_groups(zz, o["group_slot"]), "group sweep %d combine" % seed)
