"""GPU parity for the MXFP8 dispatch (EP_MXFP8_E4M3) and the FP16 I/O path
(EP_F16 dispatch, ep_combine_f16), against the oracle.

Bar: MXFP8 codes and E8M0 bytes bit-exact, the MXFP8 dequantisation
bit-exact, fp16 rows bit-exact; the fp16 combine within
|gpu - ref| <= 8e-3 * max(|ref|, 1e-3) element-wise, infinities matching.
"""
import numpy as np
import pytest
import torch

import oracle
from combine_moe_layout_amd import binding as B
from combine_moe_layout_amd import workloads as W
from test_gpu_parity import dev_bf16, gpu_layout, layout_to_host, note, sample_tokens

pytestmark = pytest.mark.gpu

REL_TOL = 8e-3
ABS_FLOOR = 1e-3


def dev_f16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.float16)


def host_f16_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def assert_close_f16(gpu_bits, ref_bits, what):
    g = gpu_bits.view(np.float16).astype(np.float64)
    r = ref_bits.view(np.float16).astype(np.float64)
    assert not np.isnan(g).any(), "%s: NaN in the output" % what
    inf = np.isinf(r)
    assert (np.isinf(g) == inf).all() and (g[inf] == r[inf]).all(), "%s: infinities differ" % what
    err = np.abs(g[~inf] - r[~inf])
    lim = REL_TOL * np.maximum(np.abs(r[~inf]), ABS_FLOOR)
    assert (err <= lim).all(), "%s: %d elements beyond tolerance" % (what, int((err > lim).sum()))
    rel = float((err / np.maximum(np.abs(r[~inf]), ABS_FLOOR)).max()) if err.size else 0.0
    note("%s: max rel err %.3e, %d infinities" % (what, rel, int(inf.sum())))


def _mx_special_rows(H, n=12, seed=5):
    """Rows with wide dynamic range, exact powers of two, block maxima that
    saturate, tiny (bf16 subnormal) and all-zero blocks."""
    g = np.random.default_rng(seed)
    rows = []
    for scale in (2.0 ** -130, 2.0 ** -120, 2.0 ** -60, 1e-3, 1.0, 255.75, 448.0, 500.0, 3.0e5,
                  2.0 ** 100, 2.0 ** 124, 0.0)[:n]:
        r = (g.standard_normal(H) * scale).astype(np.float32)
        r[::37] = 0.0
        r[1::32] = scale
        r[5::64] = -scale * 1.9
        rows.append(W.float32_to_bf16_bits(r))
    return np.stack(rows)


def _mx_dispatch(x_bits, lay, H, fill=0x5A, sfill=0xA5):
    R = lay.num_recv_rows
    q = torch.full((R, H), fill, dtype=torch.uint8, device="cuda")
    s = torch.full((R, H // 32), sfill, dtype=torch.uint8, device="cuda")
    B.ep_dispatch(dev_bf16(x_bits), lay, B.EP_MXFP8_E4M3, q, s)
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()


# --------------------------------------------------------------------------- MXFP8 dispatch
@pytest.mark.parametrize("name,T,H", [("dsv3", 256, None), ("large", 512, None), ("lowlat", None, None),
                                       ("dsv3", 37, 128), ("dsv3", 50, 384), ("dsv3", 9, 16512),
                                       ("skewed", 100, 7168)])
def test_dispatch_mxfp8(name, T, H):
    wl = W.make(name, T=T, H=H)
    note("MXFP8 dispatch %s T=%d H=%d cap=%d" % (name, wl.T, wl.H, wl.cap))
    ol = oracle.layout(wl.topk_idx, wl.E, wl.G, wl.cap)
    lay = gpu_layout(wl.topk_idx, wl.E, wl.G, wl.cap)
    q, s = _mx_dispatch(wl.x_bits, lay, wl.H)
    oq, os_ = oracle.dispatch_mxfp8(wl.x_bits, ol["slot_idx"], ol["num_recv_rows"])
    used = np.zeros(ol["num_recv_rows"], bool)
    used[ol["slot_idx"][ol["slot_idx"] >= 0]] = True
    assert (q[used] == oq[used]).all(), "codes differ"
    assert (s[used] == os_[used]).all(), "E8M0 bytes differ"
    assert (q[~used] == 0x5A).all() and (s[~used] == 0xA5).all()


def test_dispatch_mxfp8_special_blocks():
    H = 1024
    x = _mx_special_rows(H)
    T = x.shape[0]
    idx = np.stack([np.arange(4) * 3 + t % 3 for t in range(T)]).astype(np.int64)  # 4 experts each
    ol = oracle.layout(idx, 12, 1, 0)
    lay = gpu_layout(idx, 12, 1, 0)
    q, s = _mx_dispatch(x, lay, H)
    oq, os_ = oracle.dispatch_mxfp8(x, ol["slot_idx"], ol["num_recv_rows"])
    assert (q == oq).all() and (s == os_).all()
    note("MXFP8 special blocks: scale bytes %d..%d" % (int(s.min()), int(s.max())))


def test_dispatch_mxfp8_full_size_sampled():
    wl = W.make("dsv3")
    ol = oracle.layout(wl.topk_idx, wl.E, wl.G, 0)
    lay = gpu_layout(wl.topk_idx, wl.E, wl.G, 0, with_src=False)
    q, s = _mx_dispatch(wl.x_bits, lay, wl.H)
    assert (layout_to_host(lay)["slot_idx"] == ol["slot_idx"]).all()
    for t in sample_tokens(wl.T, 48):
        oq, os_ = oracle.quantize_token_mxfp8(wl.x_bits[t])
        rows = ol["slot_idx"][t]
        assert (q[rows] == oq).all() and (s[rows] == os_).all(), "token %d" % t


@pytest.mark.parametrize("T,H", [(1, 7168), (64, 7168), (128, 4096), (200, 1024)])
def test_layout_dispatch_fused_mxfp8(T, H):
    wl = W.make("lowlat", T=T, H=H)
    ol = oracle.layout(wl.topk_idx, wl.E, wl.G, wl.cap)
    lay = B.EpLayout(T, wl.k, wl.E, wl.G, wl.cap)
    R = lay.num_recv_rows
    q = torch.full((R, H), 0x5A, dtype=torch.uint8, device="cuda")
    s = torch.full((R, H // 32), 0xA5, dtype=torch.uint8, device="cuda")
    B.ep_layout_dispatch(torch.from_numpy(wl.topk_idx).cuda(), lay, dev_bf16(wl.x_bits),
                         B.EP_MXFP8_E4M3, q, s)
    torch.cuda.synchronize()
    assert (layout_to_host(lay)["slot_idx"] == ol["slot_idx"]).all()
    oq, os_ = oracle.dispatch_mxfp8(wl.x_bits, ol["slot_idx"], R)
    used = np.zeros(R, bool)
    used[ol["slot_idx"][ol["slot_idx"] >= 0]] = True
    qh, sh = q.cpu().numpy(), s.cpu().numpy()
    assert (qh[used] == oq[used]).all() and (sh[used] == os_[used]).all()
    assert (qh[~used] == 0x5A).all() and (sh[~used] == 0xA5).all()


def test_dequant_mxfp8_matches_oracle():
    """Dispatch's own rows, plus rows at the ends of the E8M0 range (bytes 0,
    1, 254 and 255, the NaN byte that makes its block 0x7FC0)."""
    H = 1024
    x = _mx_special_rows(H)
    qs = [oracle.quantize_token_mxfp8(r) for r in x]
    q = np.stack([a for a, _ in qs])
    s = np.stack([b for _, b in qs])
    g = np.random.default_rng(9)
    q_ext = g.integers(0, 256, (4, H)).astype(np.uint8)
    q_ext[(q_ext & 0x7F) == 0x7F] = 0x38
    s_ext = np.resize(np.array([0, 1, 254, 255, 127], np.uint8), (4, H // 32)).astype(np.uint8)
    q, s = np.concatenate([q, q_ext]), np.concatenate([s, s_ext])
    y = torch.empty((q.shape[0], H), dtype=torch.bfloat16, device="cuda")
    B.ep_dequant_mxfp8(torch.from_numpy(q).cuda(), torch.from_numpy(s).cuda(), y)
    torch.cuda.synchronize()
    got = y.view(torch.int16).cpu().numpy().view(np.uint16)
    assert (got == oracle.dequant_mxfp8(q, s)).all()


def test_dispatch_mxfp8_to_groups():
    wl = W.make("dsv3", T=256)
    o = oracle.group_layout(wl.topk_idx, None, wl.E, wl.G)
    gl = B.EpGroupLayout(wl.T, wl.k, wl.E, wl.G)
    B.ep_get_group_layout(torch.from_numpy(wl.topk_idx).cuda(), None, gl)
    q, s = _mx_dispatch(wl.x_bits, gl, wl.H)
    used = o["rows_used"]
    oq, os_ = oracle.dispatch_mxfp8(wl.x_bits, o["group_slot"], gl.num_recv_rows)
    assert (q[:used] == oq[:used]).all() and (s[:used] == os_[:used]).all()


# --------------------------------------------------------------------------- FP16 I/O
def _f16_rows(R, H, seed, scale=1.0):
    g = np.random.default_rng(seed)
    return (g.standard_normal((R, H)) * scale).astype(np.float16).view(np.uint16)


@pytest.mark.parametrize("name,T,H", [("tiny", None, None), ("skewed", 300, None), ("lowlat", None, None),
                                       ("dsv3", 70, 24), ("dsv3", 9, 16392)])
def test_dispatch_f16_is_a_bit_copy(name, T, H):
    wl = W.make(name, T=T, H=H)
    x = _f16_rows(wl.T, wl.H, 3)
    ol = oracle.layout(wl.topk_idx, wl.E, wl.G, wl.cap)
    lay = gpu_layout(wl.topk_idx, wl.E, wl.G, wl.cap)
    R = lay.num_recv_rows
    recv = torch.empty((R, wl.H), dtype=torch.float16, device="cuda")
    recv.view(torch.int16).fill_(0x1357)
    B.ep_dispatch(dev_f16(x), lay, B.EP_F16, recv)
    got = host_f16_bits(recv)
    want = oracle.dispatch_bf16(x, ol["slot_idx"], R)  # a 2-byte row copy, format-blind
    used = np.zeros(R, bool)
    used[ol["slot_idx"][ol["slot_idx"] >= 0]] = True
    assert (got[used] == want[used]).all() and (got[~used] == 0x1357).all()


@pytest.mark.parametrize("name,T,H,scale", [("tiny", None, None, 1.0), ("dsv3", 256, None, 1.0),
                                             ("large", 300, None, 100.0), ("lowlat", None, None, 1.0),
                                             ("dsv3", 40, 24, 1.0), ("dsv3", 9, 16512, 1.0),
                                             ("skewed", 64, 7168, 2.0 ** -14),
                                             # prefill-sized, packed 1024-lane workgroups, ragged tail
                                             ("large", 1001, None, 1.0), ("dsv3", 1029, 1024, 1.0)])
def test_combine_f16_random_rows(name, T, H, scale):
    wl = W.make(name, T=T, H=H)
    lay = gpu_layout(wl.topk_idx, wl.E, wl.G, wl.cap)
    sl = layout_to_host(lay)["slot_idx"]
    y = _f16_rows(lay.num_recv_rows, wl.H, 4, scale)
    out = torch.empty((wl.T, wl.H), dtype=torch.float16, device="cuda")
    B.ep_combine_f16(dev_f16(y), torch.from_numpy(wl.topk_weights).cuda(), lay, out)
    torch.cuda.synchronize()
    assert_close_f16(host_f16_bits(out), oracle.combine_f16(y, wl.topk_weights, sl),
                     "fp16 combine %s T=%d H=%d scale %g" % (name, wl.T, wl.H, scale))


def test_combine_f16_overflow_and_subnormals():
    T, k, H, E = 64, 4, 256, 16
    g = np.random.default_rng(12)
    idx = np.stack([g.permutation(E)[:k] for _ in range(T)]).astype(np.int64)
    lay = gpu_layout(idx, E, 1, 0)
    sl = layout_to_host(lay)["slot_idx"]
    R = lay.num_recv_rows
    y = np.empty((R, H), np.float16)
    y[:, :64] = 40000.0                                    # four rows of 40000 overflow
    y[:, 64:128] = g.choice([-1.0, 1.0], (R, 64)) * 2.0 ** -24 * g.integers(1, 1024, (R, 64))
    y[:, 128:] = g.standard_normal((R, 128)).astype(np.float16)
    w = np.ones((T, k), np.float32)
    w[::2] = 0.25                                          # even tokens: 4 * 0.25 * 40000, finite
    yb = y.view(np.uint16)
    out = torch.empty((T, H), dtype=torch.float16, device="cuda")
    B.ep_combine_f16(dev_f16(yb), torch.from_numpy(w).cuda(), lay, out)
    torch.cuda.synchronize()
    got, ref = host_f16_bits(out), oracle.combine_f16(yb, w, sl)
    assert_close_f16(got, ref, "fp16 combine, overflow and subnormals")
    assert np.isinf(got[1::2, :64].view(np.float16)).all() and np.isfinite(got[::2, :64].view(np.float16)).all()
    # sums of subnormals and small integers of 2**-24 are exact in fp32: bit-exact here
    assert (got[:, 64:128] == ref[:, 64:128]).all()


def test_f16_path_round_trip_is_exact():
    """fp16 dispatch, identity experts, fp16 combine with weights summing to
    one: every token comes back unchanged (up to the sign of zero)."""
    wl = W.make("dsv3", T=512, H=2048)
    x = _f16_rows(wl.T, wl.H, 6)
    lay = gpu_layout(wl.topk_idx, wl.E, wl.G, 0)
    R = lay.num_recv_rows
    recv = torch.empty((R, wl.H), dtype=torch.float16, device="cuda")
    B.ep_dispatch(dev_f16(x), lay, B.EP_F16, recv)
    out = torch.empty((wl.T, wl.H), dtype=torch.float16, device="cuda")
    B.ep_combine_f16(recv, torch.from_numpy(wl.topk_weights).cuda(), lay, out)
    torch.cuda.synchronize()
    got = host_f16_bits(out)
    assert ((got & 0x7FFF) == (x & 0x7FFF)).all()


def test_combine_f16_full_size_sampled():
    wl = W.make("dsv3")
    lay = gpu_layout(wl.topk_idx, wl.E, wl.G, 0, with_src=False)
    sl = layout_to_host(lay)["slot_idx"]
    y = _f16_rows(lay.num_recv_rows, wl.H, 7)
    out = torch.empty((wl.T, wl.H), dtype=torch.float16, device="cuda")
    B.ep_combine_f16(dev_f16(y), torch.from_numpy(wl.topk_weights).cuda(), lay, out)
    torch.cuda.synchronize()
    toks = sample_tokens(wl.T, 48)
    ref = oracle.combine_f16_tokens(y, wl.topk_weights, sl, toks)
    assert_close_f16(host_f16_bits(out)[toks], ref, "fp16 combine full size (sampled)")
