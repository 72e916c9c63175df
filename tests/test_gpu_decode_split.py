"""GPU parity of the decode-sized combines, where one token is spread over up to
8 workgroups (batches of at most 4096 (token, k) pairs, one token per
workgroup otherwise): bf16, fp16, FP8, MXFP8 and the unit-weight group
combine, against the oracle.

The cases set every split count from 1 to 8, slices that end inside a row,
rows that still loop (hidden 16512 over two 1024-lane slices) and the longest
row (hidden 65536, eight full slices).  Outputs start as NaN, so a column no
slice writes fails.  Bar: |gpu - ref| <= 8e-3 * max(|ref|, 1e-3) element-wise.
"""
import numpy as np
import pytest
import torch

import oracle
from combine_moe_layout_amd import binding as B
from combine_moe_layout_amd import workloads as W
from test_gpu_dedup import gpu_group_layout
from test_gpu_mx_f16 import _f16_rows, assert_close_f16, dev_f16, host_f16_bits
from test_gpu_parity import assert_close_bf16, dev_bf16, gpu_layout, host_bits, note

pytestmark = pytest.mark.gpu

# (tokens, hidden, top-k): workgroups per token = min(8, 256 // T, hidden / 512)
CASES = [(1, 7168, 8), (2, 1024, 8), (5, 16512, 8), (31, 7168, 8), (32, 1664, 8), (33, 7168, 6),
         (64, 2048, 8), (100, 7168, 8), (128, 7168, 8), (129, 7168, 8), (16, 65536, 8),
         (3, 65536, 9), (256, 7168, 8), (7, 1152, 3),
         (64, 4096, 1), (100, 2048, 2), (200, 7168, 4), (40, 640, 5),
         (384, 7168, 8), (512, 4096, 8)]   # whole-token form without a split, up to 4096 pairs

NAN_BF16, NAN_F16 = 0x7FC0, 0x7E00


def _case(T, H, k):
    return W.custom(T=T, H=H, E=64, k=k, G=8, seed=T + k)


def _unit_code_rows(R, H, seed, mx):
    """E4M3 codes of either sign with magnitudes up to 7.5 and scales 2^-3 ..
    2^0, so decoded values are of the order of real expert outputs.  These
    tests check which workgroup covers which columns; the wide-range arithmetic
    of the code combines is tested on its own, and with terms this size the
    fp32 sums stay far inside the bar even where the terms cancel."""
    g = np.random.default_rng(seed)
    q = (g.integers(0, 0x50, (R, H)) | (g.integers(0, 2, (R, H)) << 7)).astype(np.uint8)
    if mx:
        return q, g.integers(124, 127, (R, H // 32)).astype(np.uint8)
    sc = np.exp2(g.integers(-3, 0, (R, H // 128))) * (1 + g.random((R, H // 128)))
    return q, sc.astype(np.float32)


def _out(T, H, f16=False):
    bits = np.full((T, H), NAN_F16 if f16 else NAN_BF16, np.uint16)
    return dev_f16(bits) if f16 else dev_bf16(bits)


@pytest.mark.parametrize("T,H,k", CASES)
def test_decode_combine_bf16(T, H, k):
    wl = _case(T, H, k)
    note("decode combine bf16 T=%d H=%d k=%d" % (T, H, k))
    ol = oracle.layout(wl.topk_idx, wl.E, wl.G, 0)
    lay = gpu_layout(wl.topk_idx, wl.E, wl.G, 0, with_src=False)
    y = W.random_expert_outputs(wl.R, H, seed=T)
    out = _out(T, H)
    B.ep_combine(dev_bf16(y), torch.from_numpy(wl.topk_weights).cuda(), lay, out)
    torch.cuda.synchronize()
    assert_close_bf16(host_bits(out), oracle.combine(y, wl.topk_weights, ol["slot_idx"]),
                      "decode combine T=%d H=%d k=%d" % (T, H, k))


@pytest.mark.parametrize("T,H,k", CASES)
def test_decode_combine_f16(T, H, k):
    wl = _case(T, H, k)
    note("decode combine fp16 T=%d H=%d k=%d" % (T, H, k))
    ol = oracle.layout(wl.topk_idx, wl.E, wl.G, 0)
    lay = gpu_layout(wl.topk_idx, wl.E, wl.G, 0, with_src=False)
    y = _f16_rows(wl.R, H, seed=T)
    out = _out(T, H, f16=True)
    B.ep_combine_f16(dev_f16(y), torch.from_numpy(wl.topk_weights).cuda(), lay, out)
    torch.cuda.synchronize()
    assert_close_f16(host_f16_bits(out), oracle.combine_f16(y, wl.topk_weights, ol["slot_idx"]),
                     "decode combine fp16 T=%d H=%d k=%d" % (T, H, k))


@pytest.mark.parametrize("mx", [False, True], ids=["fp8", "mxfp8"])
@pytest.mark.parametrize("T,H,k", CASES)
def test_decode_combine_codes(T, H, k, mx):
    wl = _case(T, H, k)
    note("decode combine %s T=%d H=%d k=%d" % ("mxfp8" if mx else "fp8", T, H, k))
    ol = oracle.layout(wl.topk_idx, wl.E, wl.G, 0)
    lay = gpu_layout(wl.topk_idx, wl.E, wl.G, 0, with_src=False)
    q, sc = _unit_code_rows(wl.R, H, T, mx)
    out = _out(T, H)
    fn = B.ep_combine_mxfp8 if mx else B.ep_combine_fp8
    fn(torch.from_numpy(q).cuda(), torch.from_numpy(sc).cuda(),
       torch.from_numpy(wl.topk_weights).cuda(), lay, out)
    torch.cuda.synchronize()
    ref = (oracle.combine_mxfp8 if mx else oracle.combine_fp8)(q, sc, wl.topk_weights, ol["slot_idx"])
    assert_close_bf16(host_bits(out), ref, "decode combine codes T=%d H=%d k=%d" % (T, H, k))


@pytest.mark.parametrize("T,H,k", CASES)
def test_decode_combine_groups(T, H, k):
    wl = _case(T, H, k)
    note("decode group combine T=%d H=%d k=%d" % (T, H, k))
    o = oracle.group_layout(wl.topk_idx, None, wl.E, wl.G)
    gl, _, _ = gpu_group_layout(wl.topk_idx, None, wl.E, wl.G, meta=False)
    z = W.random_expert_outputs(gl.num_recv_rows, H, seed=T + 1)
    out = _out(T, H)
    B.ep_combine_groups(dev_bf16(z), gl, out)
    torch.cuda.synchronize()
    assert_close_bf16(host_bits(out), oracle.combine_groups(z, o["group_slot"]),
                      "decode group combine T=%d H=%d k=%d" % (T, H, k))


def test_split_and_unsplit_results_are_identical():
    """The split changes which workgroup sums a column, not the sum: 128 tokens
    (two workgroups per token) agree bit for bit with the same 128 tokens plus
    an unrouted 129th (one workgroup per token), whose layout gives the first
    128 tokens the same receive rows."""
    H, k = 7168, 8
    wl = W.custom(T=129, H=H, E=64, k=k, G=8, seed=11)
    idx = wl.topk_idx.copy()
    idx[128] = -1
    lay129 = gpu_layout(idx, wl.E, wl.G, 0, with_src=False)
    lay128 = gpu_layout(np.ascontiguousarray(idx[:128]), wl.E, wl.G, 0, with_src=False)
    assert np.array_equal(lay128.slot_idx.cpu().numpy(), lay129.slot_idx.cpu().numpy()[:128])
    y = W.random_expert_outputs(lay129.num_recv_rows, H, seed=12)
    w = torch.from_numpy(wl.topk_weights).cuda()
    out129, out128 = _out(129, H), _out(128, H)
    B.ep_combine(dev_bf16(y), w, lay129, out129)
    B.ep_combine(dev_bf16(np.ascontiguousarray(y[:lay128.num_recv_rows])), w[:128].contiguous(),
                 lay128, out128)
    torch.cuda.synchronize()
    got128, got129 = host_bits(out128), host_bits(out129)
    assert np.array_equal(got128, got129[:128])
    assert (got129[128] == 0).all()
