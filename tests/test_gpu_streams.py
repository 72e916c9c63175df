"""Calls on different buffers may run concurrently: the library keeps no
mutable state of its own, so two independent paths (layout, FP8 dispatch,
identity expert, combine) enqueued on two streams at once give, bit for bit,
what each gives alone.  Both streams keep the default priority."""
import numpy as np
import pytest
import torch

from combine_moe_layout_amd import binding as B
from combine_moe_layout_amd import workloads as W

pytestmark = pytest.mark.gpu


def _path_buffers(name, seed, T, H):
    wl = W.make(name, T=T, H=H, seed=seed)
    dev = torch.device("cuda")
    lay = B.EpLayout(wl.T, wl.k, wl.E, wl.G, wl.cap, device=dev)
    R = lay.num_recv_rows
    bufs = dict(
        wl=wl, lay=lay,
        idx=torch.from_numpy(wl.topk_idx).to(dev),
        x=torch.from_numpy(wl.x_bits.view(np.int16)).to(dev).view(torch.bfloat16),
        w=torch.from_numpy(wl.topk_weights).to(dev),
        q=torch.zeros((R, wl.H), dtype=torch.uint8, device=dev),
        s=torch.zeros((R, wl.H // 128), dtype=torch.float32, device=dev),
        y=torch.zeros((R, wl.H), dtype=torch.bfloat16, device=dev),
        out=torch.zeros((wl.T, wl.H), dtype=torch.bfloat16, device=dev))
    return bufs


def _run(b, stream):
    B.ep_get_layout(b["idx"], b["lay"], stream)
    B.ep_dispatch(b["x"], b["lay"], B.EP_FP8_E4M3, b["q"], b["s"], stream)
    B.ep_dequant_fp8(b["q"], b["s"], b["y"], stream)
    B.ep_combine(b["y"], b["w"], b["lay"], b["out"], stream)


def _snapshot(b):
    return [t.cpu().numpy().copy() for t in (b["lay"].slot_idx, b["lay"].num_tokens_per_expert,
                                             b["lay"].expert_offsets, b["q"], b["s"],
                                             b["out"].view(torch.int16))]


def _clear(b):
    for key in ("q", "s", "y", "out"):
        b[key].zero_()
    b["lay"].slot_idx.zero_()


def test_two_streams_match_sequential(reps=3):
    a = _path_buffers("dsv3", 1, 2048, 7168)
    b = _path_buffers("skewed", 2, 1500, 4096)   # skewed routing, FP8 dispatch here too
    print("[gpu-streams] dsv3 T=2048 and skewed T=1500 on two streams", flush=True)
    cur = torch.cuda.current_stream()
    _run(a, cur)
    _run(b, cur)
    torch.cuda.synchronize()
    want_a, want_b = _snapshot(a), _snapshot(b)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for r in range(reps):
        _clear(a)
        _clear(b)
        torch.cuda.synchronize()
        _run(a, s1)
        _run(b, s2)
        torch.cuda.synchronize()
        for got, want in zip(_snapshot(a) + _snapshot(b), want_a + want_b):
            assert np.array_equal(got, want), "concurrent run %d differs from the sequential one" % r
