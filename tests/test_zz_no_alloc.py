"""ep_get_layout_noalloc: the layout with the library's fixed per-GPU
workspace, for callers that cannot allocate at call time.

Checked through the C ABI (ctypes) against ep_get_layout on the same inputs:
every output array identical, over two calls in a row whose second input is
smaller (the array keeps the first call's contents), on the two-launch path
and on the one-launch decode path; sizes beyond the array are refused before
any launch.
"""
import ctypes

import numpy as np
import pytest
import torch

from combine_moe_layout_amd import binding as B
from combine_moe_layout_amd import workloads as W

pytestmark = pytest.mark.gpu


def note(msg):
    print("[gpu-noalloc] " + msg, flush=True)


def _arrays(lay: B.EpLayout) -> dict:
    torch.cuda.synchronize()
    return {k: getattr(lay, k).cpu().numpy() for k in (
        "num_tokens_per_expert", "expert_offsets", "num_tokens_per_group", "slot_idx",
        "error_flags")} | ({"recv_src": lay.recv_src.cpu().numpy()} if lay.recv_src is not None else {})


def _both(idx: np.ndarray, E: int, G: int, cap: int) -> None:
    T, k = idx.shape
    ti = torch.from_numpy(np.ascontiguousarray(idx, np.int64)).cuda()
    ref = B.EpLayout(T, k, E, G, cap, with_recv_src=True)
    got = B.EpLayout(T, k, E, G, cap, with_recv_src=True)
    for lay in (ref, got):
        lay.recv_src.fill_(-1)
        lay.slot_idx.fill_(-7)
    B.ep_get_layout(ti, ref)
    # straight through the C ABI, the library's own workspace
    rc = B.lib().ep_get_layout_noalloc(ti.data_ptr() if ti.numel() else None,
                                       ctypes.byref(got.struct),
                                       torch.cuda.current_stream().cuda_stream)
    assert rc == B.EP_OK, rc
    a, b = _arrays(ref), _arrays(got)
    for key in a:
        assert a[key].shape == b[key].shape and (a[key] == b[key]).all(), key


def test_noalloc_layout_matches_ep_get_layout_twice_smaller_second():
    wl = W.make("dsv3")
    note("noalloc: dsv3 (65536 pairs, two launches), then 5400 pairs E=255 k=9")
    _both(wl.topk_idx, wl.E, wl.G, 0)
    g = np.random.default_rng(3)
    _both(g.integers(-1, 255, (600, 9)).astype(np.int64), 255, 5, 0)


def test_noalloc_layout_decode_and_padded():
    wl = W.make("lowlat")
    note("noalloc: decode batch padded, then a smaller padded batch with drops")
    _both(wl.topk_idx, wl.E, wl.G, wl.cap)
    g = np.random.default_rng(4)
    _both(g.integers(0, 8, (50, 4)).astype(np.int64), 8, 2, 3)


def test_noalloc_layout_large_then_small_with_bad_ids():
    wl = W.make("large")
    note("noalloc: large (393216 pairs), then 3000 pairs with bad ids")
    _both(wl.topk_idx, wl.E, wl.G, 0)
    g = np.random.default_rng(5)
    _both(g.integers(-3, 40, (1500, 2)).astype(np.int64), 32, 4, 0)


def test_noalloc_refuses_sizes_beyond_its_array():
    # 2^21 pairs at E = 1024 need about 4.2 MB of workspace, above the 4 MiB array;
    # refused on the host, so the fake pointers are never read
    lay = B.ep_layout_t()
    assert B.lib().ep_layout_init(ctypes.byref(lay), 262144, 8, 1024, 8, 0) == B.EP_OK
    assert B.ep_layout_workspace_bytes(262144, 8, 1024) > B.EP_NOALLOC_SCRATCH_BYTES
    fake = 1 << 20
    lay.num_tokens_per_expert = lay.expert_offsets = lay.num_tokens_per_group = fake
    lay.slot_idx = lay.error_flags = fake
    assert B.lib().ep_get_layout_noalloc(fake, ctypes.byref(lay), None) == -4


def test_noalloc_layout_under_graph_capture():
    """Recorded in a HIP graph (the allocation-free entry point's first use
    case) and replayed several times, with eager calls on other inputs
    between the replays: every replay equals ep_get_layout on the recorded
    input.  The array's address is looked up by the eager calls before the
    capture; the recording only holds kernel launches."""
    wl = W.make("dsv3")
    T, k = wl.T, wl.k
    ti = torch.from_numpy(wl.topk_idx).cuda()
    ref = B.EpLayout(T, k, wl.E, wl.G, 0)
    B.ep_get_layout(ti, ref)
    want = _arrays(ref)
    lay = B.EpLayout(T, k, wl.E, wl.G, 0)
    B.ep_get_layout_noalloc(ti, lay)  # eager first call on this device
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            B.ep_get_layout_noalloc(ti, lay)
    torch.cuda.synchronize()
    g = np.random.default_rng(9)
    for rep in range(4):
        lay.slot_idx.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = _arrays(lay)
        for key in want:
            assert (got[key] == want[key]).all(), (rep, key)
        # eager calls on another input overwrite the shared array between replays
        other = g.integers(-1, 64, (3000, 6)).astype(np.int64)
        _both(other, 64, 8, 0)
    note("noalloc under graph capture: 4 replays equal to ep_get_layout")
