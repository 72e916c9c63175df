"""GPU parity of FP8 dispatch with the MN-major (transposed) scale layout,
EP_SCALES_MN_MAJOR: the same E4M3 codes and scale values as the oracle, with
scale c of receive row r stored at c * R + r.  Every path that writes scales
is covered -- the dispatch kernel (contiguous and padded layouts, drops,
masked entries, rows that loop, several tokens per workgroup), the one-launch
decode path and its two-launch fallback, and dispatch to the groups of a
dedup layout -- plus the full DeepSeek-V3-style size, sampled.  The
conversion entry point ep_scales_to_mn_major is checked against the transpose
it defines and against the flag's output.

The bar is that of every dispatch: codes and scale bits identical to the
oracle's (its scales in the MN-major layout, oracle.scales_mn_major), and
every entry of a row that no slot names left as it was.
"""
import numpy as np
import pytest
import torch

import oracle
from combine_moe_layout_amd import binding as B
from combine_moe_layout_amd import workloads as W
from test_gpu_parity import dev_bf16, gpu_layout, layout_to_host, note, sample_tokens

pytestmark = pytest.mark.gpu

MN = B.EP_SCALES_MN_MAJOR
FP8_KINDS = [B.EP_FP8_E4M3, B.EP_FP8_E4M3_POW2, B.EP_MXFP8_E4M3]
SENTINEL = 0xA5


def _oracle_dispatch(dtype, x_bits, slot_idx, R):
    if dtype == B.EP_MXFP8_E4M3:
        return oracle.dispatch_mxfp8(x_bits, slot_idx, R)
    if dtype == B.EP_FP8_E4M3_POW2:
        return oracle.dispatch_fp8_pow2(x_bits, slot_idx, R)
    return oracle.dispatch_fp8(x_bits, slot_idx, R)


def _buffers(dtype, R, H):
    """Codes [R, H] and MN-major scales ([H/32, R] bytes or [H/128, R] fp32),
    both filled with a sentinel byte pattern."""
    q = torch.full((R, H), SENTINEL, dtype=torch.uint8, device="cuda")
    if dtype == B.EP_MXFP8_E4M3:
        s = torch.full((H // 32, R), SENTINEL, dtype=torch.uint8, device="cuda")
    else:
        s = torch.empty((H // 128, R), dtype=torch.float32, device="cuda")
        s.view(torch.uint8).fill_(SENTINEL)
    return q, s


def _scale_bytes(s: torch.Tensor) -> np.ndarray:
    """MN-major scales as [entries per row, R, bytes per entry]."""
    h = s.cpu().numpy()
    return h.view(np.uint8).reshape(h.shape[0], h.shape[1], h.dtype.itemsize)


def _check(dtype, x_bits, slot_idx, q, s, what):
    torch.cuda.synchronize()
    R = q.shape[0]
    used = np.zeros(R, bool)
    used[slot_idx[slot_idx >= 0]] = True
    oq, os_ = _oracle_dispatch(dtype, x_bits, slot_idx, R)
    qh = q.cpu().numpy()
    assert (qh[used] == oq[used]).all(), "%s: codes" % what
    assert (qh[~used] == SENTINEL).all(), "%s: codes of unused rows" % what
    sb = _scale_bytes(s)                                          # [c, R, bytes]
    ob = oracle.scales_mn_major(os_)                              # the oracle's, MN-major
    ob = ob.view(np.uint8).reshape(sb.shape)
    assert (sb[:, used] == ob[:, used]).all(), "%s: scales" % what
    assert (sb[:, ~used] == SENTINEL).all(), "%s: scales of unused rows" % what
    note("%s: %d rows used of %d" % (what, int(used.sum()), R))


CASES = [
    # name, T, H, cap override (None = the workload's), mask fraction
    ("dsv3", 300, 1024, None, 0.0),
    ("dsv3", 300, 1024, 0, 0.08),      # masked entries
    ("skewed", 257, 512, 24, 0.0),     # padded, hot experts overflow: drops
    ("dsv3", 37, 128, None, 0.0),      # several tokens per workgroup
    ("dsv3", 9, 16512, None, 0.0),     # the row loops over the workgroup
    ("large", 200, 4096, None, 0.0),   # k = 6 with the shared expert
]


@pytest.mark.parametrize("dtype", FP8_KINDS)
@pytest.mark.parametrize("case", range(len(CASES)))
def test_dispatch_scales_mn_major(case, dtype):
    name, T, H, cap, mask = CASES[case]
    wl = W.make(name, T=T, H=H)
    idx = wl.topk_idx.copy()
    if mask:
        idx[np.random.default_rng(case).random(idx.shape) < mask] = -1
    cap = wl.cap if cap is None else cap
    note("MN-major scales: %s T=%d H=%d cap=%d dtype %d" % (name, T, H, cap, dtype))
    ol = oracle.layout(idx, wl.E, wl.G, cap)
    lay = gpu_layout(idx, wl.E, wl.G, cap)
    assert (layout_to_host(lay)["slot_idx"] == ol["slot_idx"]).all()
    q, s = _buffers(dtype, lay.num_recv_rows, H)
    B.ep_dispatch(dev_bf16(wl.x_bits), lay, dtype | MN, q, s)
    _check(dtype, wl.x_bits, ol["slot_idx"], q, s, "%s/%d" % (name, dtype))


@pytest.mark.parametrize("dtype", FP8_KINDS)
@pytest.mark.parametrize("T,cap", [(64, 128), (200, 0), (600, 0)])
def test_layout_dispatch_scales_mn_major(T, cap, dtype):
    """ep_layout_dispatch: one launch up to 2048 pairs, the two-launch path above."""
    wl = W.make("lowlat", T=T, H=2048)
    note("fused MN-major scales: T=%d cap=%d dtype %d (pairs %d)" % (T, cap, dtype, T * wl.k))
    ol = oracle.layout(wl.topk_idx, wl.E, wl.G, cap)
    lay = B.EpLayout(T, wl.k, wl.E, wl.G, cap)
    q, s = _buffers(dtype, lay.num_recv_rows, 2048)
    B.ep_layout_dispatch(torch.from_numpy(wl.topk_idx).cuda(), lay, dev_bf16(wl.x_bits), dtype | MN, q, s)
    assert (layout_to_host(lay)["slot_idx"] == ol["slot_idx"]).all()
    _check(dtype, wl.x_bits, ol["slot_idx"], q, s, "fused T=%d" % T)


@pytest.mark.parametrize("dtype", [B.EP_FP8_E4M3, B.EP_MXFP8_E4M3])
def test_group_dispatch_scales_mn_major(dtype):
    """Dispatch to the groups of a dedup layout (R = T * min(k, G) rows)."""
    wl = W.make("skewed", T=400, H=1024)
    o = oracle.group_layout(wl.topk_idx, None, wl.E, wl.G)
    gl = B.EpGroupLayout(wl.T, wl.k, wl.E, wl.G)
    B.ep_get_group_layout(torch.from_numpy(wl.topk_idx).cuda(), None, gl)
    q, s = _buffers(dtype, gl.num_recv_rows, wl.H)
    B.ep_dispatch(dev_bf16(wl.x_bits), gl, dtype | MN, q, s)
    torch.cuda.synchronize()
    assert (gl.slot_idx.cpu().numpy() == o["group_slot"]).all()
    _check(dtype, wl.x_bits, o["group_slot"], q, s, "groups")


@pytest.mark.parametrize("dtype", [B.EP_FP8_E4M3, B.EP_MXFP8_E4M3])
def test_dispatch_scales_mn_major_full_size_sampled(dtype):
    """T=8192, H=7168, 256 experts, top-8: the launch the benchmark times with
    its MN-major option.  Every receive row is used, so the whole scale array
    is checked against the row-major call's (itself bit-exact to the oracle in
    the other tests), and sampled tokens against the oracle directly."""
    wl = W.make("dsv3")
    ol = oracle.layout(wl.topk_idx, wl.E, wl.G, 0)
    lay = gpu_layout(wl.topk_idx, wl.E, wl.G, 0, with_src=False)
    R, H = lay.num_recv_rows, wl.H
    x = dev_bf16(wl.x_bits)
    q, s = _buffers(dtype, R, H)
    B.ep_dispatch(x, lay, dtype | MN, q, s)
    q_row = torch.empty_like(q)
    s_row = torch.empty((R, s.shape[0]), dtype=s.dtype, device="cuda")
    B.ep_dispatch(x, lay, dtype, q_row, s_row)
    torch.cuda.synchronize()
    assert torch.equal(q, q_row), "codes differ from the row-major call"
    assert torch.equal(s.view(torch.uint8).view(s.shape[0], R, -1).transpose(0, 1).contiguous(),
                       s_row.view(torch.uint8).view(R, s.shape[0], -1)), "scales differ"
    slots = layout_to_host(lay)["slot_idx"]
    assert (slots == ol["slot_idx"]).all()
    sh = _scale_bytes(s)
    for t in sample_tokens(wl.T, 32):
        quant = oracle.quantize_token_mxfp8 if dtype == B.EP_MXFP8_E4M3 else oracle.quantize_token_fp8
        oq, os_ = quant(wl.x_bits[t])
        ob = np.ascontiguousarray(os_).view(np.uint8).reshape(sh.shape[0], sh.shape[2])
        for r in slots[t]:
            assert (q[r].cpu().numpy() == oq).all(), "token %d codes" % t
            assert (sh[:, r, :] == ob).all(), "token %d scales" % t


# --------------------------------------------------------------------------- conversion
CONVERSION_SHAPES = [
    # rows, H, byte offset of both buffers.  The 16-byte path needs H % 512 == 0,
    # rows % 4 == 0 (fp32) or % 16 == 0 (E8M0) and 16-byte aligned buffers;
    # every other shape takes the one-store-per-entry path.
    (1, 128, 0), (63, 7168, 0), (65, 896, 0), (1000, 8320, 0), (4099, 1024, 0), (130, 65536, 0),
    (64, 7168, 0), (1024, 7168, 0), (4112, 2048, 0), (48, 65536, 0), (260, 1536, 0),
    (1024, 7168, 4),                 # 4-byte aligned only: the scalar path at a 16-byte shape
]


@pytest.mark.parametrize("dtype", [B.EP_FP8_E4M3, B.EP_MXFP8_E4M3])
@pytest.mark.parametrize("rows,H,offset", CONVERSION_SHAPES)
def test_scales_to_mn_major_is_the_transpose(rows, H, offset, dtype):
    """ep_scales_to_mn_major on arbitrary bit patterns: exactly the transpose.
    Shapes cover one row, ragged row tiles (64 rows for fp32, 128 for E8M0
    bytes), rows wider than one column tile (65 words at H=8320), the widest
    rows (512 words), and both store paths."""
    per_row = H // 32 if dtype == B.EP_MXFP8_E4M3 else H // 128
    g = np.random.default_rng(rows * 7 + H + offset)
    mx = dtype == B.EP_MXFP8_E4M3
    src = (g.integers(0, 256, size=(rows, per_row), dtype=np.uint8) if mx else
           g.integers(0, 2**32, size=(rows, per_row), dtype=np.uint32))
    n_bytes = src.nbytes
    # byte buffers with the data starting `offset` bytes in
    sbuf = torch.zeros(n_bytes + 16, dtype=torch.uint8, device="cuda")
    sbuf[offset:offset + n_bytes] = torch.from_numpy(src.reshape(-1).view(np.uint8)).cuda()
    dbuf = torch.full((n_bytes + 16,), SENTINEL, dtype=torch.uint8, device="cuda")
    et = torch.uint8 if mx else torch.float32
    s_view = sbuf[offset:offset + n_bytes].view(et).view(rows, per_row)
    d_view = dbuf[offset:offset + n_bytes].view(et).view(per_row, rows)
    note("scale conversion rows=%d H=%d offset=%d dtype %d" % (rows, H, offset, dtype))
    B.ep_scales_to_mn_major(s_view, H, dtype, d_view)
    torch.cuda.synchronize()
    got = dbuf.cpu().numpy()
    assert (got[:offset] == SENTINEL).all() and (got[offset + n_bytes:] == SENTINEL).all()
    got = got[offset:offset + n_bytes].view(src.dtype).reshape(per_row, rows)
    assert (got == oracle.scales_mn_major(src)).all()


@pytest.mark.parametrize("dtype", FP8_KINDS)
def test_dispatch_then_conversion_matches_the_flag(dtype):
    """Row-major dispatch followed by the conversion gives, on every used row,
    the scales the MN-major dispatch writes (full DeepSeek-V3-style size)."""
    wl = W.make("dsv3")
    lay = gpu_layout(wl.topk_idx, wl.E, wl.G, 0, with_src=False)
    R, H = lay.num_recv_rows, wl.H
    x = dev_bf16(wl.x_bits)
    q, s_flag = _buffers(dtype, R, H)
    B.ep_dispatch(x, lay, dtype | MN, q, s_flag)
    s_row = torch.empty((R, s_flag.shape[0]), dtype=s_flag.dtype, device="cuda")
    B.ep_dispatch(x, lay, dtype, q, s_row)
    s_conv = torch.empty_like(s_flag)
    B.ep_scales_to_mn_major(s_row, H, dtype, s_conv)
    torch.cuda.synchronize()
    # every receive row is used at this size (no masks, contiguous layout)
    assert int((lay.slot_idx >= 0).sum()) == R
    assert torch.equal(s_conv.view(torch.uint8), s_flag.view(torch.uint8))
