"""GPU parity at the library's limits: the largest hidden size (EP_MAX_HIDDEN
= 65536, rows longer than a workgroup: every kernel loops over the row, and a
token's scales fill the LDS staging) and the largest top-k (EP_MAX_TOPK = 64,
the combine's generic path), for every dispatch dtype and every combine.
Same bar as the other parity tests."""
import numpy as np
import pytest
import torch

import oracle
from combine_moe_layout_amd import binding as B
from combine_moe_layout_amd import workloads as W
from test_gpu_mx_f16 import assert_close_f16, dev_f16, host_f16_bits
from test_gpu_parity import assert_close_bf16, dev_bf16, gpu_layout, host_bits, layout_to_host, note

pytestmark = pytest.mark.gpu

HMAX = B.EP_MAX_HIDDEN
KMAX = B.EP_MAX_TOPK


def _dispatch_check(wl, lay, ol, dtype):
    R, H = lay.num_recv_rows, wl.H
    used = np.zeros(R, bool)
    used[ol["slot_idx"][ol["slot_idx"] >= 0]] = True
    x = dev_bf16(wl.x_bits)
    if dtype == B.EP_BF16:
        recv = torch.zeros((R, H), dtype=torch.bfloat16, device="cuda")
        B.ep_dispatch(x, lay, dtype, recv)
        got = host_bits(recv)
        assert (got[used] == oracle.dispatch_bf16(wl.x_bits, ol["slot_idx"], R)[used]).all()
        return got, None
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
    assert (sh[used].view(np.uint8) == os_[used].view(np.uint8)).all(), "scales"
    return qh, sh


@pytest.mark.parametrize("dtype", [B.EP_BF16, B.EP_FP8_E4M3, B.EP_FP8_E4M3_POW2, B.EP_MXFP8_E4M3])
def test_dispatch_at_max_hidden(dtype):
    wl = W.custom(6, HMAX, 16, 4, G=4, seed=3)
    note("dispatch H=%d dtype %d" % (HMAX, dtype))
    ol = oracle.layout(wl.topk_idx, 16, 4, 0)
    lay = gpu_layout(wl.topk_idx, 16, 4, 0)
    _dispatch_check(wl, lay, ol, dtype)


def test_combines_at_max_hidden():
    wl = W.custom(6, HMAX, 16, 4, G=4, seed=4)
    lay = gpu_layout(wl.topk_idx, 16, 4, 0)
    sl = layout_to_host(lay)["slot_idx"]
    R, w = lay.num_recv_rows, torch.from_numpy(wl.topk_weights).cuda()
    y = W.random_expert_outputs(R, HMAX, seed=5)
    out = torch.empty((6, HMAX), dtype=torch.bfloat16, device="cuda")
    B.ep_combine(dev_bf16(y), w, lay, out)
    torch.cuda.synchronize()
    assert_close_bf16(host_bits(out), oracle.combine(y, wl.topk_weights, sl), "combine H=65536")
    # FP8 expert outputs
    q, s = oracle.dispatch_fp8(W.random_expert_outputs(R, HMAX, seed=6), np.arange(R, dtype=np.int32)[:, None], R)
    B.ep_combine_fp8(torch.from_numpy(q).cuda(), torch.from_numpy(s).cuda(), w, lay, out)
    torch.cuda.synchronize()
    assert_close_bf16(host_bits(out), oracle.combine_fp8(q, s, wl.topk_weights, sl), "FP8 combine H=65536")
    # fp16 rows
    yh = np.random.default_rng(7).standard_normal((R, HMAX)).astype(np.float16).view(np.uint16)
    oh = torch.empty((6, HMAX), dtype=torch.float16, device="cuda")
    B.ep_combine_f16(dev_f16(yh), w, lay, oh)
    torch.cuda.synchronize()
    assert_close_f16(host_f16_bits(oh), oracle.combine_f16(yh, wl.topk_weights, sl), "fp16 combine H=65536")


def test_fused_and_group_paths_at_max_hidden():
    wl = W.custom(5, HMAX, 32, 8, G=4, seed=8)
    ol = oracle.layout(wl.topk_idx, 32, 4, 0)
    lay = B.EpLayout(5, 8, 32, 4)
    R = lay.num_recv_rows
    q = torch.zeros((R, HMAX), dtype=torch.uint8, device="cuda")
    s = torch.zeros((R, HMAX // 128), dtype=torch.float32, device="cuda")
    B.ep_layout_dispatch(torch.from_numpy(wl.topk_idx).cuda(), lay, dev_bf16(wl.x_bits), B.EP_FP8_E4M3, q, s)
    torch.cuda.synchronize()
    assert (layout_to_host(lay)["slot_idx"] == ol["slot_idx"]).all()
    oq, os_ = oracle.dispatch_fp8(wl.x_bits, ol["slot_idx"], R)
    assert (q.cpu().numpy() == oq).all() and (s.cpu().numpy().view(np.uint32) == os_.view(np.uint32)).all()
    # per-group dedup: group layout, dispatch to the groups, group combine
    o = oracle.group_layout(wl.topk_idx, None, 32, 4)
    gl = B.EpGroupLayout(5, 8, 32, 4)
    B.ep_get_group_layout(torch.from_numpy(wl.topk_idx).cuda(), None, gl)
    z = W.random_expert_outputs(gl.num_recv_rows, HMAX, seed=9)
    out = torch.empty((5, HMAX), dtype=torch.bfloat16, device="cuda")
    B.ep_combine_groups(dev_bf16(z), gl, out)
    torch.cuda.synchronize()
    assert (gl.slot_idx.cpu().numpy() == o["group_slot"]).all()
    assert_close_bf16(host_bits(out), oracle.combine_groups(z, o["group_slot"]), "group combine H=65536")


@pytest.mark.parametrize("dtype", [B.EP_BF16, B.EP_FP8_E4M3, B.EP_MXFP8_E4M3])
def test_max_topk_dispatch_and_combine(dtype):
    """k = 64: the combine's generic path (no compile-time top-k) and 64 row
    stores per dispatched token."""
    T, H, E = 40, 1024, 128
    g = np.random.default_rng(10)
    idx = np.stack([g.permutation(E)[:KMAX] for _ in range(T)]).astype(np.int64)
    idx[g.random(idx.shape) < 0.1] = -1
    wl = W.custom(T, H, E, KMAX, G=2, fp8=dtype != B.EP_BF16, seed=11)
    wl.topk_idx = idx
    ol = oracle.layout(idx, E, 2, 0)
    lay = gpu_layout(idx, E, 2, 0)
    note("k=64 dispatch dtype %d" % dtype)
    _dispatch_check(wl, lay, ol, dtype)
    y = W.random_expert_outputs(lay.num_recv_rows, H, seed=12)
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    B.ep_combine(dev_bf16(y), torch.from_numpy(wl.topk_weights).cuda(), lay, out)
    torch.cuda.synchronize()
    assert_close_bf16(host_bits(out), oracle.combine(y, wl.topk_weights, ol["slot_idx"]), "combine k=64")
