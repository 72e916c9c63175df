"""GPU parity of ep_combine_mxfp8 (combine of MXFP8 expert outputs: E4M3 codes
with one E8M0 byte per 32 channels) against the oracle.

Bar: |gpu - ref| <= 8e-3 * max(|ref|, 1e-3) element-wise (fp32 against fp64
sums), bit-exact where every output is a single exact term, NaN where the
oracle's is NaN.
"""
import numpy as np
import pytest
import torch

import oracle
from combine_moe_layout_amd import binding as B
from combine_moe_layout_amd import workloads as W
from test_gpu_parity import assert_close_bf16, dev_bf16, gpu_layout, host_bits, note, sample_tokens

pytestmark = pytest.mark.gpu


def _random_mx_rows(R, H, seed, lo=115, hi=132):
    """Random codes (no NaN) and scale bytes 2^-12 .. 2^4, the spread of the
    FP8 combine's test scales: a much wider spread makes the weighted sums of
    random-signed rows cancel far below their terms, where any fp32 sum is off
    by more than the tolerance relative to the result."""
    g = np.random.default_rng(seed)
    q = g.integers(0, 256, (R, H)).astype(np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x38            # no NaN codes
    sc = g.integers(lo, hi, (R, H // 32)).astype(np.uint8)
    return q, sc


def _combine_mx_gpu(q, sc, w, lay, H):
    out = torch.empty((lay.num_tokens, H), dtype=torch.bfloat16, device="cuda")
    B.ep_combine_mxfp8(torch.from_numpy(q).cuda(), torch.from_numpy(sc).cuda(),
                       torch.from_numpy(np.ascontiguousarray(w, np.float32)).cuda(), lay, out)
    torch.cuda.synchronize()
    return host_bits(out)


@pytest.mark.parametrize("name,T,H", [("dsv3", 200, None), ("lowlat", None, None), ("large", 400, None),
                                       ("dsv3", 64, 128), ("dsv3", 21, 16512), ("dsv3", 37, 384)])
def test_combine_mxfp8_random_outputs(name, T, H):
    """Top-k 8 and 6, padded rows (lowlat), rows that loop (H=16512) and short
    rows shared by several tokens in a workgroup (H=128, 384)."""
    wl = W.make(name, T=T, H=H)
    note("combine_mxfp8 %s T=%d H=%d k=%d cap=%d" % (name, wl.T, wl.H, wl.k, wl.cap))
    q, sc = _random_mx_rows(wl.R, wl.H, seed=3)
    ol = oracle.layout(wl.topk_idx, wl.E, wl.G, wl.cap)
    lay = gpu_layout(wl.topk_idx, wl.E, wl.G, wl.cap, with_src=False)
    assert_close_bf16(_combine_mx_gpu(q, sc, wl.topk_weights, lay, wl.H),
                      oracle.combine_mxfp8(q, sc, wl.topk_weights, ol["slot_idx"]), "combine_mxfp8 %s" % name)


@pytest.mark.parametrize("name,T,H", [("dsv3", 600, 7168), ("dsv3", 520, 4608), ("dsv3", 520, 7296),
                                       ("dsv3", 520, 3200), ("dsv3", 513, 16512), ("large", 700, None)])
def test_combine_mxfp8_prefill_widths(name, T, H):
    """Prefill-sized batches (more than 4096 pairs) at widths whose rows are
    split over several workgroups per token in different ways (whole, ragged
    and partly filled slices).  Codes with the sign bit clear and softmax
    weights, so that no sum cancels below the tolerance's reach."""
    wl = W.make(name, T=T, H=H)
    assert wl.T * wl.k > 4096 and (wl.topk_weights >= 0).all()
    note("combine_mxfp8 prefill %s T=%d H=%d k=%d" % (name, wl.T, wl.H, wl.k))
    q, sc = _random_mx_rows(wl.R, wl.H, seed=13)
    q &= 0x7F
    q[q == 0x7F] = 0x38
    ol = oracle.layout(wl.topk_idx, wl.E, wl.G, wl.cap)
    lay = gpu_layout(wl.topk_idx, wl.E, wl.G, wl.cap, with_src=False)
    assert_close_bf16(_combine_mx_gpu(q, sc, wl.topk_weights, lay, wl.H),
                      oracle.combine_mxfp8(q, sc, wl.topk_weights, ol["slot_idx"]),
                      "combine_mxfp8 prefill %s H=%d" % (name, wl.H))


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5, 9])
def test_combine_mxfp8_other_topk(k):
    """The compile-time top-k sizes and the generic path (k = 3, 5, 9), with
    masked pairs."""
    wl = W.custom(T=120, H=512, E=32, k=k, G=4, seed=k)
    idx = wl.topk_idx.copy()
    idx[np.random.default_rng(k).random(idx.shape) < 0.1] = -1
    note("combine_mxfp8 k=%d" % k)
    q, sc = _random_mx_rows(wl.R, wl.H, seed=k)
    ol = oracle.layout(idx, wl.E, wl.G, 0)
    lay = gpu_layout(idx, wl.E, wl.G, 0, with_src=False)
    assert_close_bf16(_combine_mx_gpu(q, sc, wl.topk_weights, lay, wl.H),
                      oracle.combine_mxfp8(q, sc, wl.topk_weights, ol["slot_idx"]), "combine_mxfp8 k=%d" % k)


def test_combine_mxfp8_decodes_codes_and_scales_exactly():
    """One-hot weights: each output is one code times 2^(byte - 127), formed
    exactly on both sides and rounded once to bf16 -- every non-NaN code, scale
    bytes from 0 (2^-127, a subnormal fp32 scale) to 254 (products past the
    bf16 range overflow to infinity on both) -- so the bits must match, zeros
    of either sign aside."""
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    H, R = 256, 16
    q = np.resize(codes, (R, H)).astype(np.uint8)
    sc = np.resize(np.array([0, 1, 2, 100, 120, 127, 128, 140, 160, 200, 230, 250, 254], np.uint8),
                   (R, H // 32)).astype(np.uint8)
    w = np.zeros((R, 2), np.float32)
    w[:, 0] = 1.0
    idx = np.stack([np.arange(R), np.full(R, -1)], 1).astype(np.int64)
    lay = gpu_layout(idx, R, 1, 1, with_src=False)   # padded, capacity 1: row t is expert t's
    ol = oracle.layout(idx, R, 1, 1)
    got = _combine_mx_gpu(q, sc, w, lay, H)
    ref = oracle.combine_mxfp8(q, sc, w, ol["slot_idx"])
    gf, rf = W.bf16_bits_to_float32(got), W.bf16_bits_to_float32(ref)
    same = (got == ref) | (np.isnan(gf) & np.isnan(rf)) | ((gf == 0) & (rf == 0))
    assert same.all(), [(r, c, hex(got[r, c]), hex(ref[r, c])) for r, c in np.argwhere(~same)[:4]]


def test_combine_mxfp8_nan_scale():
    """Scale byte 255 (NaN in E8M0) turns its block's columns NaN, like the oracle."""
    R, H = 4, 128
    q = np.full((R, H), 0x38, np.uint8)
    sc = np.full((R, H // 32), 127, np.uint8)
    sc[1, 2] = 255
    idx = np.arange(R, dtype=np.int64).reshape(R, 1)
    lay = gpu_layout(idx, R, 1, 1, with_src=False)
    got = W.bf16_bits_to_float32(_combine_mx_gpu(q, sc, np.ones((R, 1), np.float32), lay, H))
    ref = W.bf16_bits_to_float32(oracle.combine_mxfp8(q, sc, np.ones((R, 1), np.float32),
                                                      oracle.layout(idx, R, 1, 1)["slot_idx"]))
    assert (np.isnan(got) == np.isnan(ref)).all() and np.isnan(got[1, 64:96]).all()
    assert (got[~np.isnan(ref)] == ref[~np.isnan(ref)]).all()


def test_whole_path_mxfp8_combine_full_size():
    """dsv3 at full size: MXFP8 dispatch, identity experts kept in MXFP8 (the
    receive codes and scale bytes are the expert outputs), MXFP8 combine;
    sampled tokens through the oracle's own chain."""
    wl = W.make("dsv3")
    note("whole path with MXFP8 combine, dsv3 full size")
    lay = gpu_layout(wl.topk_idx, wl.E, wl.G, 0, with_src=False)
    q = torch.empty((wl.R, wl.H), dtype=torch.uint8, device="cuda")
    s = torch.empty((wl.R, wl.H // 32), dtype=torch.uint8, device="cuda")
    B.ep_dispatch(dev_bf16(wl.x_bits), lay, B.EP_MXFP8_E4M3, q, s)
    out = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda")
    B.ep_combine_mxfp8(q, s, torch.from_numpy(wl.topk_weights).cuda(), lay, out)
    got = host_bits(out)
    ol = oracle.layout(wl.topk_idx, wl.E, wl.G, 0)
    toks = sample_tokens(wl.T, 48)
    ref = np.empty((toks.size, wl.H), np.uint16)
    for i, t in enumerate(toks):
        qt, st = oracle.quantize_token_mxfp8(wl.x_bits[t])
        local = np.where(ol["slot_idx"][t] >= 0, 0, -1).astype(np.int32).reshape(1, -1)
        ref[i] = oracle.combine_mxfp8(qt.reshape(1, -1), st.reshape(1, -1), wl.topk_weights[t:t + 1], local)[0]
    assert_close_bf16(got[toks], ref, "whole path MXFP8 combine")
