"""Pins for the oracle's variants: power-of-two FP8 scales and FP8 combine (CPU only)."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from combine_moe_layout_amd import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
bf = workloads.float32_to_bf16_bits
unbf = workloads.bf16_bits_to_float32


def _ev(expr):
    return float(eval(expr, {"__builtins__": {}}, {}))


def _decode_all(q):
    table = np.array([oracle.e4m3_decode(c) for c in range(256)])
    return table[q]


def test_pow2_golden_blocks():
    with open(os.path.join(GOLDEN, "fp8_pow2_block.json")) as f:
        blocks = json.load(f)["blocks"]
    for blk in blocks:
        x = np.zeros(128, np.float32)
        want = np.zeros(128, np.uint8)
        for i, (expr, code) in enumerate(blk["x"]):
            x[i] = _ev(expr)
            want[i] = int(code, 16)
        assert (unbf(bf(x)) == x).all(), blk["why"]
        q, s = oracle.quantize_token_fp8_pow2(bf(x))
        assert s[0] == np.float32(_ev(blk["scale"])), (blk["why"], s[0])
        assert (q == want).all(), (blk["why"], [(i, hex(a), hex(b)) for i, (a, b) in enumerate(zip(q, want)) if a != b])


@pytest.mark.parametrize("name", ["dsv3", "large"])
def test_pow2_scale_is_the_smallest_power_of_two(name):
    wl = workloads.make(name, T=64)
    H = wl.H
    for t in range(wl.T):
        q, s = oracle.quantize_token_fp8_pow2(wl.x_bits[t])
        x = unbf(wl.x_bits[t]).reshape(H // 128, 128).astype(np.float64)
        a = np.maximum(np.abs(x).max(1), float(np.float32(1e-4)))
        m, e = np.frexp(s.astype(np.float64))
        assert (m == 0.5).all()                          # a power of two
        assert (448.0 * s >= a).all() and (448.0 * s / 2 < a).all()
        # codes are torch's E4M3 cast of the exact rescale x / s (clamped)
        v = np.clip(x / s[:, None].astype(np.float64), -448, 448).astype(np.float32)
        ref = torch.from_numpy(v.reshape(-1)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert (q == ref).all()
        # error bound of round-to-nearest E4M3 with scale s
        deq = _decode_all(q).reshape(H // 128, 128) * s[:, None]
        assert (np.abs(deq - x) <= 2.0 ** -4 * np.abs(x) + 2.0 ** -10 * s[:, None] + 1e-30).all()


def test_pow2_dispatch_copies():
    wl = workloads.make("dsv3", T=20, H=512)
    lay = oracle.layout(wl.topk_idx, wl.E, wl.G, 0)
    q, s = oracle.dispatch_fp8_pow2(wl.x_bits, lay["slot_idx"], wl.R)
    for t in range(wl.T):
        q1, s1 = oracle.quantize_token_fp8_pow2(wl.x_bits[t])
        rows = lay["slot_idx"][t]
        assert (q[rows] == q1).all() and (s[rows] == s1).all()


def test_combine_fp8_golden():
    with open(os.path.join(GOLDEN, "combine_fp8_tiny.json")) as f:
        c = json.load(f)
    H = c["H"]
    R = len(c["rows"])
    q = np.zeros((R, H), np.uint8)
    sc = np.zeros((R, H // 128), np.float32)
    for r, row in enumerate(c["rows"]):
        for ch, code in row["codes"]:
            q[r, ch] = int(code, 16)
        sc[r, :] = _ev(row["scale"])
    slot = np.array(c["slot_idx"], np.int32)
    w = np.array([[_ev(v) for v in row] for row in c["topk_weights"]], np.float32)
    out = oracle.combine_fp8(q, sc, w, slot)
    for o in c["out"]:
        for ch, bits in o["bits"]:
            assert out[o["token"], ch] == int(bits, 16), (o["why"], ch, hex(out[o["token"], ch]))


def test_combine_fp8_one_hot_is_the_dequantisation():
    g = np.random.default_rng(2)
    R, H, T, k = 150, 256, 40, 3
    q = g.integers(0, 256, (R, H)).astype(np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x10          # no NaN codes
    sc = (g.random((R, H // 128)) + 0.1).astype(np.float32)
    slot = g.permutation(R)[: T * k].reshape(T, k).astype(np.int32)
    w = np.zeros((T, k), np.float32)
    pick = g.integers(0, k, T)
    w[np.arange(T), pick] = 1.0
    out = oracle.combine_fp8(q, sc, w, slot)
    want = oracle.dequant_fp8(q, sc)[slot[np.arange(T), pick]]
    assert ((out == want) | (((out | want) & 0x7FFF) == 0)).all()


def test_combine_fp8_vs_float64_sum():
    g = np.random.default_rng(4)
    R, H, T, k = 300, 384, 64, 8
    q = g.integers(0, 256, (R, H)).astype(np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x22
    sc = (g.random((R, H // 128)) * 0.01 + 1e-3).astype(np.float32)
    slot = g.integers(-1, R, (T, k)).astype(np.int32)
    w = g.random((T, k)).astype(np.float32)
    out = unbf(oracle.combine_fp8(q, sc, w, slot)).astype(np.float64)
    vals = _decode_all(q) * np.repeat(sc.astype(np.float64), 128, 1)
    ref = np.zeros((T, H))
    for j in range(k):
        m = slot[:, j] >= 0
        ref[m] += w[m, j:j + 1].astype(np.float64) * vals[slot[m, j]]
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -126))) - 7)
    assert (np.abs(out - ref) <= 0.5 * ulp * (1 + 1e-9)).all()


def test_fp8_round_trip_through_fp8_combine():
    """FP8 dispatch, identity experts kept in FP8, weights summing to 1: the
    output is within the E4M3 bound of x."""
    for quant, disp in ((oracle.quantize_token_fp8, oracle.dispatch_fp8),
                        (oracle.quantize_token_fp8_pow2, oracle.dispatch_fp8_pow2)):
        wl = workloads.make("dsv3", T=24, H=1024)
        lay = oracle.layout(wl.topk_idx, wl.E, wl.G, 0)
        q, s = disp(wl.x_bits, lay["slot_idx"], wl.R)
        out = unbf(oracle.combine_fp8(q, s, wl.topk_weights, lay["slot_idx"])).astype(np.float64)
        x = unbf(wl.x_bits).astype(np.float64)
        assert (np.abs(out - x) <= (2.0 ** -4 + 2.0 ** -7) * np.abs(x) + 2.0 ** -9 * s.max()).all()
