"""Pins of the oracle's MN-major scale layout (R20), CPU only.

The layout is a change of storage order with a plain definition: entry c of
receive row r at c * R + r.  Pinned against a pure-Python index loop on small
arrays of both entry sizes (fp32 scales, E8M0 bytes), and, composed with the
oracle's FP8 and MXFP8 dispatch, against the scales of each token quantised on
its own: column r of the MN-major array holds the scales of the token routed
to receive row r.
"""
import numpy as np
import pytest

import oracle
from combine_moe_layout_amd import workloads as W


def _by_loops(a):
    rows, n = a.shape
    out = [[None] * rows for _ in range(n)]
    for r in range(rows):
        for c in range(n):
            out[c][r] = a[r, c]
    return np.array(out, dtype=a.dtype).reshape(n, rows)


@pytest.mark.parametrize("rows,n", [(1, 1), (3, 5), (17, 56), (64, 2), (5, 224)])
def test_scales_mn_major_matches_index_loops(rows, n):
    g = np.random.default_rng(rows * 31 + n)
    words = g.integers(0, 2**32, size=(rows, n), dtype=np.uint32).view(np.float32)
    got = oracle.scales_mn_major(words)
    assert got.shape == (n, rows) and got.dtype == np.float32
    assert (got.view(np.uint32) == _by_loops(words.view(np.uint32))).all()
    bytes_ = g.integers(0, 256, size=(rows, n), dtype=np.uint8)
    got = oracle.scales_mn_major(bytes_)
    assert got.shape == (n, rows) and (got == _by_loops(bytes_)).all()


def test_scales_mn_major_of_no_rows():
    assert oracle.scales_mn_major(np.zeros((0, 7), np.float32)).shape == (7, 0)


@pytest.mark.parametrize("mx", [False, True])
def test_mn_major_columns_are_the_tokens_scales(mx):
    wl = W.make("dsv3", T=40, H=512)
    ol = oracle.layout(wl.topk_idx, wl.E, wl.G, 0)
    R = ol["num_recv_rows"]
    _, s = (oracle.dispatch_mxfp8 if mx else oracle.dispatch_fp8)(wl.x_bits, ol["slot_idx"], R)
    mn = oracle.scales_mn_major(s)
    quant = oracle.quantize_token_mxfp8 if mx else oracle.quantize_token_fp8
    for t in range(wl.T):
        _, ts = quant(wl.x_bits[t])
        for r in ol["slot_idx"][t]:
            col = np.ascontiguousarray(mn[:, r])
            assert (col.view(np.uint8) == np.ascontiguousarray(ts).view(np.uint8)).all(), (t, r)
