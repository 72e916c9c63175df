"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Both sides are fed from the same seeded generators and never see each
other's outputs.  The bar: layout, slots, bf16 dispatch, FP8 codes and scales
and the identity-expert dequantisation are bit-exact; combine is within
|gpu - ref| <= 8e-3 * max(|ref|, 1e-3) element-wise (the oracle sums in fp64,
the kernel in fp32; both round once to bf16).  At the workloads' full sizes
(the launch shapes the benchmark times) every receive row and every output
token is compared; the oracle's per-token calls run on several host threads.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
from combine_moe_layout_amd import binding as B
from combine_moe_layout_amd import workloads as W

pytestmark = pytest.mark.gpu

REL_TOL = 8e-3
ABS_FLOOR = 1e-3


def note(msg):
    print("[gpu-parity] " + msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "the GPU tests need an MI355X"
    B.lib()
    note("library: %s" % B.ep_version())


# --------------------------------------------------------------------------- helpers
def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def gpu_layout(idx: np.ndarray, E: int, G: int, cap: int, with_src: bool = True) -> B.EpLayout:
    T, k = idx.shape
    lay = B.EpLayout(T, k, E, G, cap, with_recv_src=with_src)
    if with_src and lay.recv_src is not None:
        lay.recv_src.fill_(-1)
    B.ep_get_layout(torch.from_numpy(np.ascontiguousarray(idx, np.int64)).cuda(), lay)
    return lay


def layout_to_host(lay: B.EpLayout) -> dict:
    torch.cuda.synchronize()
    return dict(num_tokens_per_expert=lay.num_tokens_per_expert.cpu().numpy(),
                expert_offsets=lay.expert_offsets.cpu().numpy(),
                num_tokens_per_group=lay.num_tokens_per_group.cpu().numpy(),
                slot_idx=lay.slot_idx.cpu().numpy(),
                recv_src=None if lay.recv_src is None else lay.recv_src.cpu().numpy(),
                error_flags=int(lay.error_flags.cpu()[0]))


def assert_layout_equal(g: dict, o: dict, what: str):
    for key in ("num_tokens_per_expert", "expert_offsets", "num_tokens_per_group", "slot_idx"):
        a, b = g[key], o[key]
        assert a.shape == b.shape and (a == b).all(), "%s: %s differs (first at %s)" % (
            what, key, np.argwhere(a != b)[:3].tolist())
    if g["recv_src"] is not None:
        assert (g["recv_src"] == o["recv_src"]).all(), "%s: recv_src differs" % what
    assert g["error_flags"] == o["error_flags"], "%s: flags %d vs %d" % (
        what, g["error_flags"], o["error_flags"])


def assert_close_bf16(gpu_bits: np.ndarray, ref_bits: np.ndarray, what: str) -> float:
    g = W.bf16_bits_to_float32(gpu_bits).astype(np.float64)
    r = W.bf16_bits_to_float32(ref_bits).astype(np.float64)
    assert np.isfinite(g).all(), "%s: non-finite output" % what
    err = np.abs(g - r)
    lim = REL_TOL * np.maximum(np.abs(r), ABS_FLOOR)
    bad = np.argwhere(err > lim)
    assert bad.size == 0, "%s: %d elements beyond tolerance, first %s (gpu %r ref %r)" % (
        what, len(bad), bad[0].tolist(), g[tuple(bad[0])], r[tuple(bad[0])])
    rel = float((err / np.maximum(np.abs(r), ABS_FLOOR)).max()) if err.size else 0.0
    note("%s: max rel err %.3e (tol %.0e)" % (what, rel, REL_TOL))
    return rel


def sample_tokens(T: int, n: int, seed: int = 0) -> np.ndarray:
    g = np.random.default_rng(1234 + seed)
    picks = set(g.choice(T, size=min(n, T), replace=False).tolist())
    picks.update([0, T - 1])
    return np.array(sorted(picks), np.int64)


# --------------------------------------------------------------------------- FP8 encoder
def test_fp8_encoder_exhaustive():
    """Every fp32 bit pattern of magnitude <= 448, both signs: the kernel's
    encoders (dispatch's, the software one, the conversion instruction) give
    the oracle's code."""
    top = 0x43E00000
    chunk = 1 << 26
    out = torch.empty(chunk, dtype=torch.uint8, device="cuda")
    oracle.lib()
    pool = ThreadPoolExecutor(16)
    bad = {0: 0, 1: 0, 2: 0}
    for sign in (0, 1):
        base = 0x80000000 if sign else 0
        note("fp8 encoder sweep, sign %d" % sign)
        for start in range(0, top + 1, chunk):
            n = min(chunk, top + 1 - start)
            parts = [(base + start + i, min(1 << 22, n - i)) for i in range(0, n, 1 << 22)]
            ref = np.concatenate(list(pool.map(lambda a: oracle.e4m3_encode_bits(*a), parts)))
            for method in (0, 1, 2):
                B.ep_cast_e4m3_bits(base + start, n, method, out)
                got = out[:n].cpu().numpy()
                bad[method] += int((got != ref).sum())
    pool.shutdown()
    assert bad == {0: 0, 1: 0, 2: 0}, bad


# --------------------------------------------------------------------------- layout
@pytest.mark.parametrize("name", list(W.CONFIGS))
def test_layout_named_workloads(name):
    T, H, E, G, k, cap, fp8, kind = W.CONFIGS[name]
    idx, _ = W.route(kind, T, E, k, G, seed=0)
    note("layout %s T=%d k=%d E=%d cap=%d" % (name, T, k, E, cap))
    g = layout_to_host(gpu_layout(idx, E, G, cap))
    assert_layout_equal(g, oracle.layout(idx, E, G, cap), name)


def _edge_layouts():
    g = np.random.default_rng(77)
    cases = [
        ("empty", np.zeros((0, 4), np.int64), 8, 2, 0),
        ("one pair", np.array([[0]], np.int64), 1, 1, 0),
        ("ragged 2049 pairs", g.integers(0, 16, (2049, 1)), 16, 4, 0),
        ("ragged 4097 pairs k=17", g.integers(0, 64, (241, 17)), 64, 8, 0),
        ("all to one expert", np.full((3000, 8), 5, np.int64), 256, 8, 0),
        ("masked and bad ids", g.integers(-3, 40, (1500, 6)), 32, 4, 0),
        ("all unrouted", np.full((100, 4), -1, np.int64), 16, 4, 0),
        ("E=1024", g.integers(0, 1024, (8192, 8)), 1024, 8, 0),
        ("E=3 G=3", g.integers(0, 3, (999, 2)), 3, 3, 0),
        ("k=64", g.integers(0, 128, (300, 64)), 128, 2, 0),
        ("padded overflow cap=1", g.integers(0, 8, (500, 4)), 8, 2, 1),
        ("padded overflow cap=37", g.integers(-1, 16, (2500, 3)), 16, 4, 37),
        ("padded hot expert", np.concatenate([np.zeros((700, 1)), g.integers(1, 64, (700, 5))], 1), 64, 8, 128),
        ("many chunks, few experts", g.integers(0, 4, (200000, 2)), 4, 2, 0),
        # more chunks than workgroups resident at once: the two-launch path
        ("1.1M pairs, 547 chunks", g.integers(0, 64, (140000, 8)), 64, 8, 0),
        ("1.1M pairs padded", g.integers(-1, 64, (140000, 8)), 64, 8, 20000),
        # one lane per expert in the finish scan, many batches of chunks each
        ("E=1024, 300 chunks", g.integers(0, 1024, (76800, 8)), 1024, 8, 0),
        # the extra launch that computes every chunk's bases once (chunks^2 * E
        # large), with experts that leave its last workgroup partly idle
        ("E=100, 300 chunks, bases launch", g.integers(-1, 100, (76800, 8)), 100, 10, 0),
        ("E=100, 300 chunks padded, bases launch", g.integers(0, 100, (76800, 8)), 100, 10, 5000),
        # one layout chunk, top-k <= 8: one workgroup per token
        ("one chunk: masked and bad ids", g.integers(-3, 40, (200, 6)), 32, 4, 0),
        ("one chunk: padded overflow cap=3", g.integers(-1, 16, (300, 4)), 16, 4, 3),
        ("one chunk: 2048 pairs exactly", g.integers(0, 256, (256, 8)), 256, 8, 0),
        ("one chunk: E=1024", g.integers(0, 1024, (100, 8)), 1024, 8, 0),
        ("one chunk: all to one expert, padded", np.full((200, 8), 7, np.int64), 16, 2, 100),
        # one layout chunk with top-k 9: the single-workgroup layout
        ("one chunk: k=9", g.integers(0, 64, (200, 9)), 64, 8, 0),
        # two-launch path with a count matrix (chunks x E) that is not a
        # multiple of 4, odd expert counts (parts of lanes per expert that do
        # not fill the workgroup) and many chunks per part
        ("E=253, 3 chunks, matrix 759", g.integers(0, 253, (700, 8)), 253, 11, 0),
        ("E=255, k=9, 3 chunks, matrix 765", g.integers(-1, 255, (600, 9)), 255, 5, 0),
        ("E=1, 259 chunks, matrix 259", np.zeros((530000, 1), np.int64), 1, 1, 0),
        ("E=7, 41 chunks, matrix 287", g.integers(0, 7, (10300, 8)), 7, 7, 0),
        ("E=13 padded, 21 chunks, matrix 273", g.integers(-1, 13, (5300, 8)), 13, 13, 700),
    ]
    return cases


@pytest.mark.parametrize("case", range(len(_edge_layouts())))
def test_layout_edge_cases(case):
    name, idx, E, G, cap = _edge_layouts()[case]
    idx = np.ascontiguousarray(idx, np.int64)
    note("layout edge case: %s %s" % (name, idx.shape))
    g = layout_to_host(gpu_layout(idx, E, G, cap))
    assert_layout_equal(g, oracle.layout(idx, E, G, cap), name)


def test_layout_is_deterministic():
    T, H, E, G, k, cap, fp8, kind = W.CONFIGS["skewed"]
    idx, _ = W.route(kind, T, E, k, G, seed=3)
    note("layout determinism (skewed, 5 runs)")
    first = layout_to_host(gpu_layout(idx, E, G, cap))
    for _ in range(4):
        assert_layout_equal(layout_to_host(gpu_layout(idx, E, G, cap)), first, "rerun")


# --------------------------------------------------------------------------- dispatch
def _dispatch_gpu(wl, lay, fill=None):
    R = lay.num_recv_rows
    x = dev_bf16(wl.x_bits)
    if wl.fp8:
        recv = torch.zeros((R, wl.H), dtype=torch.uint8, device="cuda")
        sc = torch.zeros((R, wl.H // 128), dtype=torch.float32, device="cuda")
        if fill is not None:
            recv.fill_(fill)
            sc.fill_(float(fill))
        B.ep_dispatch(x, lay, B.EP_FP8_E4M3, recv, sc)
        torch.cuda.synchronize()
        return recv.cpu().numpy(), sc.cpu().numpy()
    recv = torch.zeros((R, wl.H), dtype=torch.bfloat16, device="cuda")
    if fill is not None:
        recv.view(torch.int16).fill_(fill)
    B.ep_dispatch(x, lay, B.EP_BF16, recv)
    torch.cuda.synchronize()
    return host_bits(recv), None


DISPATCH_CASES = [
    # name, T, H (None = the workload's), override fp8
    ("tiny", None, None, None),
    ("skewed", 384, None, None),
    ("dsv3", 256, None, None),
    ("lowlat", None, None, None),
    ("large", 512, None, None),
    ("dsv3", 37, 128, None),      # 8 lanes per token, several tokens per workgroup
    ("dsv3", 50, 384, None),      # 24 lanes rounded to 32
    ("dsv3", 9, 16512, None),     # more vectors than one workgroup: the row loops
    ("skewed", 70, 24, None),     # bf16, 3 vectors per row
    ("skewed", 33, 16392, None),  # bf16, row loops
    ("large", 300, 4096, False),  # bf16 at the large shape
]


@pytest.mark.parametrize("case", range(len(DISPATCH_CASES)))
def test_dispatch_full_compare(case):
    name, T, H, fp8 = DISPATCH_CASES[case]
    wl = W.make(name, T=T, H=H)
    if fp8 is not None:
        wl.fp8 = fp8
    note("dispatch %s T=%d H=%d fp8=%s cap=%d" % (name, wl.T, wl.H, wl.fp8, wl.cap))
    ol = oracle.layout(wl.topk_idx, wl.E, wl.G, wl.cap)
    lay = gpu_layout(wl.topk_idx, wl.E, wl.G, wl.cap)
    fill = 0x5A if wl.fp8 else 0x1234  # rows no slot names must keep it
    q, s = _dispatch_gpu(wl, lay, fill=fill)
    used = np.zeros(ol["num_recv_rows"], bool)
    used[ol["slot_idx"][ol["slot_idx"] >= 0]] = True
    if wl.fp8:
        oq, os_ = oracle.dispatch_fp8(wl.x_bits, ol["slot_idx"], ol["num_recv_rows"])
        assert (q[used] == oq[used]).all(), "FP8 codes differ"
        assert (s[used].view(np.uint32) == os_[used].view(np.uint32)).all(), "FP8 scales differ"
        assert (q[~used] == fill).all() and (s[~used] == float(fill)).all()
    else:
        orecv = oracle.dispatch_bf16(wl.x_bits, ol["slot_idx"], ol["num_recv_rows"])
        assert (q[used] == orecv[used]).all(), "bf16 rows differ"
        assert (q[~used] == fill).all()


@pytest.mark.parametrize("name", ["dsv3", "large", "skewed"])
def test_dispatch_full_size_complete(name):
    """Every receive row at the workload's full size (the benchmark's launch
    shape): codes and scale bits (FP8) or row bits (bf16) against the oracle's
    whole dispatch."""
    wl = W.make(name)
    note("dispatch full size %s T=%d H=%d, every row" % (name, wl.T, wl.H))
    ol = oracle.layout(wl.topk_idx, wl.E, wl.G, wl.cap)
    lay = gpu_layout(wl.topk_idx, wl.E, wl.G, wl.cap, with_src=False)
    q, s = _dispatch_gpu(wl, lay)
    g_slots = layout_to_host(lay)["slot_idx"]
    assert (g_slots == ol["slot_idx"]).all()
    R = ol["num_recv_rows"]
    used = np.zeros(R, bool)
    used[ol["slot_idx"][ol["slot_idx"] >= 0]] = True
    if wl.fp8:
        oq, os_ = oracle.dispatch_fp8(wl.x_bits, ol["slot_idx"], R)
        bad = np.argwhere((q != oq).any(1) & used)
        assert bad.size == 0, "%d rows' codes differ, first row %d" % (len(bad), bad[0][0])
        bad = np.argwhere((s.view(np.uint32) != os_.view(np.uint32)).any(1) & used)
        assert bad.size == 0, "%d rows' scales differ, first row %d" % (len(bad), bad[0][0])
        note("%d rows of codes and scales identical" % used.sum())
    else:
        orecv = oracle.dispatch_bf16(wl.x_bits, ol["slot_idx"], R)
        bad = np.argwhere((q != orecv).any(1) & used)
        assert bad.size == 0, "%d rows differ, first row %d" % (len(bad), bad[0][0])
        note("%d rows identical" % used.sum())


def test_dequant_matches_oracle():
    wl = W.make("dsv3", T=128)
    note("dequant (identity expert) T=128")
    ol = oracle.layout(wl.topk_idx, wl.E, wl.G, 0)
    oq, os_ = oracle.dispatch_fp8(wl.x_bits, ol["slot_idx"], wl.R)
    oy = oracle.dequant_fp8(oq, os_)
    lay = gpu_layout(wl.topk_idx, wl.E, wl.G, 0, with_src=False)
    x = dev_bf16(wl.x_bits)
    q = torch.empty((wl.R, wl.H), dtype=torch.uint8, device="cuda")
    s = torch.empty((wl.R, wl.H // 128), dtype=torch.float32, device="cuda")
    B.ep_dispatch(x, lay, B.EP_FP8_E4M3, q, s)
    y = torch.empty((wl.R, wl.H), dtype=torch.bfloat16, device="cuda")
    B.ep_dequant_fp8(q, s, y)
    assert (host_bits(y) == oy).all()


# --------------------------------------------------------------------------- combine
COMBINE_CASES = [
    # name, T, H, k override
    ("tiny", None, None),
    ("skewed", 300, None),
    ("dsv3", 200, None),
    ("large", 400, None),
    ("lowlat", None, None),
    ("dsv3", 33, 24),      # H % 16 != 0: 8-channel lanes
    ("dsv3", 21, 16400),   # row loops
    ("dsv3", 64, 128),     # several tokens per workgroup
    # prefill-sized batches packed into 1024-lane workgroups, ragged last workgroup
    ("large", 1001, None),  # 512 lanes per token: 2 tokens per workgroup
    ("dsv3", 1027, 2048),  # 256 lanes: 4 per workgroup
    ("dsv3", 1029, 1024),  # 128 lanes: 8 per workgroup
    ("dsv3", 1100, 512),   # 64 lanes: 16 per workgroup
    ("dsv3", 1030, 3072),  # 384 lanes: does not divide 1024, one token per workgroup
]


def _combine_gpu(y_bits, w, lay, H):
    y = dev_bf16(y_bits)
    wt = torch.from_numpy(np.ascontiguousarray(w, np.float32)).cuda()
    out = torch.empty((lay.num_tokens, H), dtype=torch.bfloat16, device="cuda")
    B.ep_combine(y, wt, lay, out)
    torch.cuda.synchronize()
    return host_bits(out)


@pytest.mark.parametrize("case", range(len(COMBINE_CASES)))
def test_combine_random_expert_outputs(case):
    name, T, H = COMBINE_CASES[case]
    wl = W.make(name, T=T, H=H)
    note("combine %s T=%d H=%d k=%d" % (name, wl.T, wl.H, wl.k))
    y = W.random_expert_outputs(wl.R, wl.H, seed=5)
    ol = oracle.layout(wl.topk_idx, wl.E, wl.G, wl.cap)
    lay = gpu_layout(wl.topk_idx, wl.E, wl.G, wl.cap, with_src=False)
    got = _combine_gpu(y, wl.topk_weights, lay, wl.H)
    ref = oracle.combine(y, wl.topk_weights, ol["slot_idx"])
    assert_close_bf16(got, ref, "combine %s" % name)


@pytest.mark.parametrize("k", [1, 3, 9, 13])
def test_combine_other_topk(k):
    """k outside the compile-time set runs the general loop."""
    wl = W.custom(T=150, H=512, E=32, k=k, G=4, seed=k)
    note("combine k=%d" % k)
    y = W.random_expert_outputs(wl.R, wl.H, seed=k)
    ol = oracle.layout(wl.topk_idx, wl.E, wl.G, 0)
    lay = gpu_layout(wl.topk_idx, wl.E, wl.G, 0, with_src=False)
    assert_close_bf16(_combine_gpu(y, wl.topk_weights, lay, wl.H),
                      oracle.combine(y, wl.topk_weights, ol["slot_idx"]), "combine k=%d" % k)


def test_combine_skips_dropped_and_unrouted_pairs():
    """Padded layout with drops, unrouted pairs and NaN in every row no slot
    names: nothing from those rows reaches the output."""
    g = np.random.default_rng(8)
    T, k, E, cap, H = 400, 4, 8, 150, 256
    idx = g.integers(-1, E, (T, k)).astype(np.int64)
    w = g.random((T, k)).astype(np.float32)
    note("combine with drops and NaN rows")
    ol = oracle.layout(idx, E, 2, cap)
    assert ol["error_flags"] & 2
    y = W.random_expert_outputs(E * cap, H, seed=9)
    used = np.zeros(E * cap, bool)
    used[ol["slot_idx"][ol["slot_idx"] >= 0]] = True
    y[~used] = 0x7FC0  # NaN
    lay = gpu_layout(idx, E, 2, cap, with_src=False)
    got = _combine_gpu(y, w, lay, H)
    assert_close_bf16(got, oracle.combine(y, w, ol["slot_idx"]), "combine drops")


def test_combine_full_size_complete():
    """Every output token of the dsv3 combine (random expert outputs) against
    the oracle's fp64 sum."""
    wl = W.make("dsv3")
    note("combine full size dsv3 with random expert outputs, every token")
    y = W.random_expert_outputs(wl.R, wl.H, seed=6)
    ol = oracle.layout(wl.topk_idx, wl.E, wl.G, 0)
    lay = gpu_layout(wl.topk_idx, wl.E, wl.G, 0, with_src=False)
    got = _combine_gpu(y, wl.topk_weights, lay, wl.H)
    ref = _oracle_tokens(lambda toks: oracle.combine_tokens(y, wl.topk_weights, ol["slot_idx"], toks),
                         wl.T, wl.H)
    assert_close_bf16(got, ref, "combine dsv3 full size")


def _oracle_tokens(fn, T: int, H: int, parts: int = 16) -> np.ndarray:
    """fn(tokens) -> [len(tokens), H] bf16 bits, over all T tokens, split
    into ranges run on threads (each oracle call runs single-threaded C)."""
    bounds = np.linspace(0, T, parts + 1).astype(np.int64)
    ranges = [np.arange(bounds[i], bounds[i + 1], dtype=np.int64) for i in range(parts)]
    with ThreadPoolExecutor(parts) as ex:
        outs = list(ex.map(lambda r: fn(r) if len(r) else np.zeros((0, H), np.uint16), ranges))
    return np.concatenate(outs)


# --------------------------------------------------------------------------- whole path
@pytest.mark.parametrize("name", list(W.CONFIGS))
def test_whole_path_identity_experts(name):
    """layout -> dispatch -> identity expert -> combine at the full size, on
    the GPU; every token through the oracle's own chain."""
    wl = W.make(name)
    note("whole path %s T=%d H=%d E=%d k=%d fp8=%s cap=%d" % (
        name, wl.T, wl.H, wl.E, wl.k, wl.fp8, wl.cap))
    lay = gpu_layout(wl.topk_idx, wl.E, wl.G, wl.cap, with_src=False)
    x = dev_bf16(wl.x_bits)
    R, H = wl.R, wl.H
    if wl.fp8:
        q = torch.empty((R, H), dtype=torch.uint8, device="cuda")
        s = torch.empty((R, H // 128), dtype=torch.float32, device="cuda")
        B.ep_dispatch(x, lay, B.EP_FP8_E4M3, q, s)
        y = torch.zeros((R, H), dtype=torch.bfloat16, device="cuda")
        B.ep_dequant_fp8(q, s, y)
        del q, s
    else:
        y = torch.zeros((R, H), dtype=torch.bfloat16, device="cuda")
        B.ep_dispatch(x, lay, B.EP_BF16, y)
    out = torch.empty((wl.T, H), dtype=torch.bfloat16, device="cuda")
    B.ep_combine(y, torch.from_numpy(wl.topk_weights).cuda(), lay, out)
    got = host_bits(out)
    del y
    ol = oracle.layout(wl.topk_idx, wl.E, wl.G, wl.cap)
    chain = oracle.chain_fp8_tokens if wl.fp8 else oracle.chain_bf16_tokens
    ref = _oracle_tokens(lambda toks: chain(wl.x_bits, wl.topk_weights, ol["slot_idx"], toks),
                         wl.T, H)
    assert_close_bf16(got, ref, "whole path %s, every token" % name)
    if not wl.fp8:
        # bf16 dispatch, identity experts, weights summing to 1: x comes back
        same = (got == wl.x_bits) | (((got | wl.x_bits) & 0x7FFF) == 0)
        assert same.all()


def test_error_flags_on_gpu():
    idx = np.array([[0, 9], [1, -1], [0, 0]], np.int64)
    note("error flags")
    g = layout_to_host(gpu_layout(idx, 4, 1, 0))
    assert g["error_flags"] == 1 and g["slot_idx"][0, 1] == -1 and g["slot_idx"][1, 1] == -1
    g = layout_to_host(gpu_layout(np.zeros((5, 2), np.int64), 4, 1, 3))
    assert g["error_flags"] == 2 and (g["slot_idx"].reshape(-1)[3:] == -1).all()
    g = layout_to_host(gpu_layout(np.zeros((3, 1), np.int64), 4, 1, 0))
    assert g["error_flags"] == 0


# --------------------------------------------------------------------------- fused low-latency path
def _fused_cases():
    g = np.random.default_rng(31)
    cases = []
    wl = W.make("lowlat")
    cases.append(("lowlat (padded, FP8)", wl.topk_idx, wl.x_bits, wl.E, wl.G, wl.cap, True))
    wl = W.make("tiny")
    cases.append(("tiny (bf16)", wl.topk_idx, wl.x_bits, wl.E, wl.G, wl.cap, False))
    wl = W.make("dsv3", T=256)
    cases.append(("2048 pairs", wl.topk_idx, wl.x_bits, wl.E, wl.G, 0, True))
    cases.append(("one token, one expert", np.array([[0]], np.int64), W.draw_x(1, 256), 1, 1, 0, True))
    idx = g.integers(-3, 24, (37, 3)).astype(np.int64)
    idx[5] = [4, 4, 4]  # the same expert three times in one token
    cases.append(("masked, bad ids, duplicates, bf16 H=200", idx, W.draw_x(37, 200), 20, 4, 0, False))
    cases.append(("padded overflow cap=3", g.integers(0, 8, (60, 5)).astype(np.int64), W.draw_x(60, 384),
                  8, 2, 3, True))
    cases.append(("rows longer than a workgroup", g.integers(0, 64, (16, 8)).astype(np.int64),
                  W.draw_x(16, 16512), 64, 8, 0, True))
    # top-k above 8 in one layout chunk: the two calls' kernels instead
    cases.append(("top-k 9, one chunk", g.integers(-1, 32, (50, 9)).astype(np.int64),
                  W.draw_x(50, 256), 32, 4, 0, True))
    cases.append(("top-k 12 padded, one chunk", g.integers(0, 16, (40, 12)).astype(np.int64),
                  W.draw_x(40, 512), 16, 4, 20, True))
    # the largest one-launch batch (4096 pairs, two layout chunks), and one pair more
    wl = W.make("dsv3", T=512, H=1024)
    cases.append(("4096 pairs, the largest fused batch", wl.topk_idx, wl.x_bits, wl.E, wl.G, 0, True))
    cases.append(("4096 pairs padded with drops", wl.topk_idx, wl.x_bits, wl.E, wl.G, 12, True))
    cases.append(("4104 pairs, top-k 8: the two-call kernels", g.integers(-1, 64, (513, 8)).astype(np.int64),
                  W.draw_x(513, 512), 64, 8, 0, True))
    return cases


@pytest.mark.parametrize("case", range(len(_fused_cases())))
def test_layout_dispatch_fused_small_batches(case):
    name, idx, x_bits, E, G, cap, fp8 = _fused_cases()[case]
    T, k = idx.shape
    H = x_bits.shape[1]
    note("fused layout+dispatch: %s T=%d k=%d E=%d H=%d cap=%d fp8=%s" % (name, T, k, E, H, cap, fp8))
    lay = B.EpLayout(T, k, E, G, cap, with_recv_src=True)
    lay.recv_src.fill_(-1)
    R = lay.num_recv_rows
    x = dev_bf16(x_bits)
    if fp8:
        q = torch.full((R, H), 0x5A, dtype=torch.uint8, device="cuda")
        s = torch.full((R, H // 128), 7.0, dtype=torch.float32, device="cuda")
        B.ep_layout_dispatch(torch.from_numpy(idx).cuda(), lay, x, B.EP_FP8_E4M3, q, s)
    else:
        q = torch.empty((R, H), dtype=torch.bfloat16, device="cuda")
        q.view(torch.int16).fill_(0x1234)
        s = None
        B.ep_layout_dispatch(torch.from_numpy(idx).cuda(), lay, x, B.EP_BF16, q)
    g_lay = layout_to_host(lay)
    ol = oracle.layout(idx, E, G, cap)
    assert_layout_equal(g_lay, ol, name)
    used = np.zeros(R, bool)
    used[ol["slot_idx"][ol["slot_idx"] >= 0]] = True
    if fp8:
        oq, os_ = oracle.dispatch_fp8(x_bits, ol["slot_idx"], R)
        qh, sh = q.cpu().numpy(), s.cpu().numpy()
        assert (qh[used] == oq[used]).all() and (sh[used].view(np.uint32) == os_[used].view(np.uint32)).all()
        assert (qh[~used] == 0x5A).all() and (sh[~used] == 7.0).all()
    else:
        orecv = oracle.dispatch_bf16(x_bits, ol["slot_idx"], R)
        qh = host_bits(q)
        assert (qh[used] == orecv[used]).all() and (qh[~used] == 0x1234).all()


def test_layout_dispatch_large_batch_takes_the_two_launch_path():
    wl = W.make("dsv3", T=1024, H=1024)
    note("ep_layout_dispatch on 8192 pairs")
    lay = B.EpLayout(wl.T, wl.k, wl.E, wl.G, 0)
    q = torch.empty((wl.R, wl.H), dtype=torch.uint8, device="cuda")
    s = torch.empty((wl.R, wl.H // 128), dtype=torch.float32, device="cuda")
    B.ep_layout_dispatch(torch.from_numpy(wl.topk_idx).cuda(), lay, dev_bf16(wl.x_bits), B.EP_FP8_E4M3, q, s)
    ol = oracle.layout(wl.topk_idx, wl.E, wl.G, 0)
    assert (layout_to_host(lay)["slot_idx"] == ol["slot_idx"]).all()
    oq, os_ = oracle.dispatch_fp8(wl.x_bits, ol["slot_idx"], wl.R)
    assert (q.cpu().numpy() == oq).all() and (s.cpu().numpy().view(np.uint32) == os_.view(np.uint32)).all()


@pytest.mark.parametrize("name,T,H,fp8", [("dsv3", None, None, True), ("skewed", 1024, None, False),
                                          ("dsv3", 300, 2048, True), ("lowlat", None, None, True),
                                          ("large", None, None, True)])
def test_layout_dispatch_read_x_ahead(name, T, H, fp8):
    """EP_READ_X_AHEAD changes where x is read from, never the results: layout
    and every receive row against the oracle.  (dsv3 and skewed read all of x
    ahead, large its first 128 MiB; the decode batch ignores the flag.)"""
    wl = W.make(name, T=T, H=H)
    note("ep_layout_dispatch | EP_READ_X_AHEAD: %s T=%d H=%d fp8=%s" % (name, wl.T, wl.H, fp8))
    lay = B.EpLayout(wl.T, wl.k, wl.E, wl.G, wl.cap)
    R = lay.num_recv_rows
    x = dev_bf16(wl.x_bits)
    ti = torch.from_numpy(wl.topk_idx).cuda()
    ol = oracle.layout(wl.topk_idx, wl.E, wl.G, wl.cap)
    used = np.zeros(R, bool)
    used[ol["slot_idx"][ol["slot_idx"] >= 0]] = True
    if fp8:
        q = torch.empty((R, wl.H), dtype=torch.uint8, device="cuda")
        s = torch.empty((R, wl.H // 128), dtype=torch.float32, device="cuda")
        B.ep_layout_dispatch(ti, lay, x, B.EP_FP8_E4M3 | B.EP_READ_X_AHEAD, q, s)
        assert_layout_equal(layout_to_host(lay), dict(ol, recv_src=None), name)
        oq, os_ = oracle.dispatch_fp8(wl.x_bits, ol["slot_idx"], R)
        qh, sh = q.cpu().numpy(), s.cpu().numpy()
        assert ((qh != oq).any(1) & used).sum() == 0
        assert ((sh.view(np.uint32) != os_.view(np.uint32)).any(1) & used).sum() == 0
    else:
        q = torch.empty((R, wl.H), dtype=torch.bfloat16, device="cuda")
        B.ep_layout_dispatch(ti, lay, x, B.EP_BF16 | B.EP_READ_X_AHEAD, q)
        assert_layout_equal(layout_to_host(lay), dict(ol, recv_src=None), name)
        orecv = oracle.dispatch_bf16(wl.x_bits, ol["slot_idx"], R)
        assert ((host_bits(q) != orecv).any(1) & used).sum() == 0
