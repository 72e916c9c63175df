"""The path recorded in a HIP graph and replayed gives the eager results.

Each replay is separated by eager work of the program's own (buffers cleared
by torch fill kernels, new input data copied in) and checked against the
eager result for the inputs of that replay.  Nothing in the path records a
memset node: the layout's flags and counts are plain kernel stores.
"""
import numpy as np
import pytest
import torch

from combine_moe_layout_amd import binding as B
from combine_moe_layout_amd import workloads as W

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16).cpu().numpy()


@pytest.mark.parametrize("name,T,H,fused", [("lowlat", None, None, True),
                                             ("lowlat", None, None, False),   # one-chunk layout
                                             ("dsv3", 1024, 1024, False)])
def test_graph_replays_match_eager(name, T, H, fused):
    print("[gpu-graph] %s T=%s H=%s fused=%s" % (name, T, H, fused), flush=True)
    wl = W.make(name, T=T, H=H)
    wl2 = W.make(name, T=T, H=H, seed=5)   # second input set, same shapes
    dev = torch.device("cuda")
    idx = torch.from_numpy(wl.topk_idx).to(dev)
    x = torch.from_numpy(wl.x_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    w = torch.from_numpy(wl.topk_weights).to(dev)
    lay = B.EpLayout(wl.T, wl.k, wl.E, wl.G, wl.cap, device=dev)
    R = lay.num_recv_rows
    q = torch.zeros((R, wl.H), dtype=torch.uint8, device=dev)
    s = torch.zeros((R, wl.H // 128), dtype=torch.float32, device=dev)
    y = torch.zeros((R, wl.H), dtype=torch.bfloat16, device=dev)
    out = torch.zeros((wl.T, wl.H), dtype=torch.bfloat16, device=dev)

    def path():
        if fused:
            B.ep_layout_dispatch(idx, lay, x, B.EP_FP8_E4M3, q, s)
        else:
            B.ep_get_layout(idx, lay)
            B.ep_dispatch(x, lay, B.EP_FP8_E4M3, q, s)
        B.ep_dequant_fp8(q, s, y)
        B.ep_combine(y, w, lay, out)

    def snapshot():
        torch.cuda.synchronize()
        return (lay.slot_idx.cpu().numpy().copy(), lay.num_tokens_per_expert.cpu().numpy().copy(),
                int(lay.error_flags.cpu()[0]), q.cpu().numpy().copy(), s.cpu().numpy().copy(),
                _bits(out).copy())

    def clear():
        for t in (q, s, y, out, lay.slot_idx, lay.num_tokens_per_expert, lay.error_flags):
            t.zero_()

    inputs = [(wl.topk_idx, wl.x_bits, wl.topk_weights), (wl2.topk_idx, wl2.x_bits, wl2.topk_weights)]
    expected = []
    for ti, xi, wi in inputs:  # eager reference for each input set, from cleared buffers
        clear()
        idx.copy_(torch.from_numpy(ti))
        x.copy_(torch.from_numpy(xi.view(np.int16)).view(torch.bfloat16))
        w.copy_(torch.from_numpy(wi))
        path()
        expected.append(snapshot())

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        path()
    for r in range(6):
        ti, xi, wi = inputs[r % 2]
        # the program's own eager work between replays
        clear()
        idx.copy_(torch.from_numpy(ti))
        x.copy_(torch.from_numpy(xi.view(np.int16)).view(torch.bfloat16))
        w.copy_(torch.from_numpy(wi))
        torch.cuda.synchronize()
        graph.replay()
        got = snapshot()
        want = expected[r % 2]
        for a, b in zip(got, want):
            assert np.array_equal(a, b), "replay %d differs from the eager result" % r


@pytest.mark.parametrize("name,T,H", [("dsv3", 1024, 1024), ("skewed", 600, 512),
                                       ("dsv3", 200, 1024)])   # one-chunk group layout
def test_graph_replays_match_eager_dedup_mxfp8(name, T, H):
    """The per-group dedup path with MXFP8 dispatch: group layout with the
    receiving side's metadata, dispatch to the groups, the MXFP8 stand-in
    expert, group combine."""
    print("[gpu-graph] dedup+mxfp8 %s T=%s H=%s" % (name, T, H), flush=True)
    wl = W.make(name, T=T, H=H)
    wl2 = W.make(name, T=T, H=H, seed=7)
    dev = torch.device("cuda")
    idx = torch.from_numpy(wl.topk_idx).to(dev)
    x = torch.from_numpy(wl.x_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    w = torch.from_numpy(wl.topk_weights).to(dev)
    gl = B.EpGroupLayout(wl.T, wl.k, wl.E, wl.G, with_recv_src=True, device=dev)
    R = gl.num_recv_rows
    ridx = torch.zeros((R, wl.k), dtype=torch.int64, device=dev)
    rw = torch.zeros((R, wl.k), dtype=torch.float32, device=dev)
    q = torch.zeros((R, wl.H), dtype=torch.uint8, device=dev)
    s = torch.zeros((R, wl.H // 32), dtype=torch.uint8, device=dev)
    z = torch.zeros((R, wl.H), dtype=torch.bfloat16, device=dev)
    out = torch.zeros((wl.T, wl.H), dtype=torch.bfloat16, device=dev)

    def path():
        B.ep_get_group_layout(idx, w, gl, ridx, rw)
        B.ep_dispatch(x, gl, B.EP_MXFP8_E4M3, q, s)
        B.ep_dequant_mxfp8(q, s, z)
        B.ep_combine_groups(z, gl, out)

    def snapshot():
        torch.cuda.synchronize()
        return tuple(t.cpu().numpy().copy() for t in (gl.slot_idx, gl.expert_offsets, gl.recv_src,
                                                      gl.error_flags, ridx, rw, q, s)) + (_bits(out).copy(),)

    def clear():
        for t in (ridx, rw, q, s, z, out, gl.slot_idx, gl.expert_offsets, gl.recv_src, gl.error_flags):
            t.zero_()

    def load(ti, xi, wi):
        idx.copy_(torch.from_numpy(ti))
        x.copy_(torch.from_numpy(xi.view(np.int16)).view(torch.bfloat16))
        w.copy_(torch.from_numpy(wi))

    inputs = [(wl.topk_idx, wl.x_bits, wl.topk_weights), (wl2.topk_idx, wl2.x_bits, wl2.topk_weights)]
    expected = []
    for inp in inputs:
        clear()
        load(*inp)
        path()
        expected.append(snapshot())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        path()
    for r in range(6):
        clear()
        load(*inputs[r % 2])
        torch.cuda.synchronize()
        graph.replay()
        for a, b in zip(snapshot(), expected[r % 2]):
            assert np.array_equal(a, b), "replay %d differs from the eager result" % r
