"""Pins for the oracle's MXFP8 and FP16 variants (CPU only).

MXFP8 (reading R18): E4M3 codes with one E8M0 scale byte per 32 channels, the
OCP Microscaling conversion.  Pinned by hand-worked blocks, torch's E8M0 and
E4M3 types (an independent implementation of both formats), the shared
exponent's defining bracket and the error bound.

FP16 (reading R19): binary16 rounding and the fp16 combine.  Pinned by
hand-worked values, numpy's float16 (decoded exhaustively, rounding on random
values and constructed ties), and exact sums.

MXFP8 combine (reading R21): a hand-worked case, the one-hot reduction to the
MXFP8 dequantisation, and a float64 sum built on torch's E4M3 and E8M0 decodes.
"""
import json
import os
from fractions import Fraction

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


def _e4m3_values(q):
    return torch.from_numpy(np.ascontiguousarray(q)).view(torch.float8_e4m3fn).double().numpy()


def _e8m0_values(b):
    return torch.from_numpy(np.ascontiguousarray(b)).view(torch.float8_e8m0fnu).double().numpy()


# --------------------------------------------------------------------------- MXFP8
def test_mxfp8_golden_blocks():
    with open(os.path.join(GOLDEN, "mxfp8_block.json")) as f:
        blocks = json.load(f)["blocks"]
    for blk in blocks:
        x = np.zeros(32, np.float32)
        want = np.zeros(32, np.uint8)
        for i, (expr, code) in enumerate(blk["x"]):
            x[i] = _ev(expr)
            want[i] = int(code, 16)
        assert (unbf(bf(x)) == x).all(), blk["why"]
        q, s = oracle.quantize_token_mxfp8(bf(x))
        assert s.tolist() == [blk["byte"]], (blk["why"], s)
        assert (q == want).all(), (blk["why"], [(i, hex(a), hex(b)) for i, (a, b) in enumerate(zip(q, want)) if a != b])


def _mx_rows(name, T=24):
    wl = workloads.make(name, T=T)
    rows = [wl.x_bits[t] for t in range(wl.T)]
    # blocks with wide dynamic range, exact powers of two and near-powers, tiny and zero blocks
    g = np.random.default_rng(5)
    H = wl.H
    for scale in (2.0 ** -120, 2.0 ** -60, 1e-3, 1.0, 255.75, 448.0, 3.0e5, 2.0 ** 100):
        r = (g.standard_normal(H) * scale).astype(np.float32)
        r[::37] = 0.0
        r[1::32] = scale                      # block maxima on the scale itself
        rows.append(bf(r))
    rows.append(np.zeros(H, np.uint16))
    return np.stack(rows)


@pytest.mark.parametrize("name", ["dsv3", "large"])
def test_mxfp8_shared_exponent_and_codes(name):
    rows = _mx_rows(name)
    H = rows.shape[1]
    for r in rows:
        q, s = oracle.quantize_token_mxfp8(r)
        x = unbf(r).astype(np.float64).reshape(H // 32, 32)
        amax = np.abs(x).max(1)
        X = _e8m0_values(s)                                   # torch's E8M0 decode: 2**(b - 127)
        assert (X == np.ldexp(1.0, s.astype(np.int64) - 127)).all()
        live = amax >= 2.0 ** -119                            # no clamp at -127 for these
        assert (amax[live] / X[live] >= 256).all() and (amax[live] / X[live] < 512).all()
        assert (s[(amax > 0) & ~live] == 0).all() and (s[amax == 0] == 0).all()
        # codes: torch's E4M3 cast of the exact rescale, clamped
        v = np.clip(x / X[:, None], -448, 448).astype(np.float32).reshape(-1)
        ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert (q == ref).all()


def test_mxfp8_error_bound_and_saturation():
    rows = _mx_rows("dsv3")
    H = rows.shape[1]
    for r in rows:
        q, s = oracle.quantize_token_mxfp8(r)
        x = unbf(r).astype(np.float64).reshape(H // 32, 32)
        X = _e8m0_values(s)[:, None]
        got = _e4m3_values(q).reshape(H // 32, 32) * X
        inside = np.abs(x) <= 448 * X
        err = np.abs(got - x)
        # half an E4M3 ulp: 2**-4 relative for normals, 2**-10 * X for subnormals
        assert (err[inside] <= (2.0 ** -4 * np.abs(x) + 2.0 ** -10 * X)[inside]).all()
        # above 448 * X the code saturates at +-448
        assert (np.abs(got[~inside]) == 448 * np.broadcast_to(X, x.shape)[~inside]).all()
        assert (np.sign(got[~inside]) == np.sign(x[~inside])).all()


def test_mxfp8_dispatch_and_dequant():
    wl = workloads.make("dsv3", T=16, H=256)
    lay = oracle.layout(wl.topk_idx, wl.E, wl.G, 0)
    R = lay["num_recv_rows"]
    q, s = oracle.dispatch_mxfp8(wl.x_bits, lay["slot_idx"], R)
    for t in range(wl.T):
        tq, ts = oracle.quantize_token_mxfp8(wl.x_bits[t])
        for slot in lay["slot_idx"][t]:
            assert (q[slot] == tq).all() and (s[slot] == ts).all()
    y = oracle.dequant_mxfp8(q, s)
    # the product decode(q) * 2**(b - 127) is exact in fp32 here, so torch's
    # single fp32 -> bf16 rounding is the reference
    prod = (_e4m3_values(q) * np.repeat(_e8m0_values(s), 32, axis=1)).astype(np.float32)
    ref = torch.from_numpy(prod).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (y == ref).all()


# --------------------------------------------------------------------------- FP16
def _f16():
    with open(os.path.join(GOLDEN, "f16_values.json")) as f:
        return json.load(f)


def test_f16_golden_values():
    g = _f16()
    for expr, bits, why in g["round"]:
        assert oracle.f16_from_double(_ev(expr)) == int(bits, 16), (expr, why)
    for bits, expr in g["decode"]:
        assert oracle.f16_to_double(int(bits, 16)) == _ev(expr), (bits, expr)


def test_f16_decode_exhaustive_against_numpy():
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = pats.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_double(int(p)) for p in pats])
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all()
    assert (got[~nan] == ref[~nan]).all()
    assert (np.signbit(got[~nan]) == np.signbit(ref[~nan])).all()


def test_f16_rounding_against_numpy():
    g = np.random.default_rng(3)
    vals = list(g.standard_normal(20000) * np.exp2(g.integers(-30, 18, 20000)))
    # exact midpoints between neighbouring binary16 values, and their neighbours
    pats = g.integers(0, 0x7BFF, 4000).astype(np.uint16)
    lo = pats.view(np.float16).astype(np.float64)
    hi = (pats + 1).astype(np.uint16).view(np.float16).astype(np.float64)
    mid = (lo + hi) / 2
    vals += list(mid) + list(-mid) + list(np.nextafter(mid, 0)) + list(np.nextafter(mid, np.inf))
    vals += [65504.0, 65519.999, 65520.0, 70000.0, 1e300, 2.0 ** -24, 2.0 ** -25, 2.0 ** -26, 0.0, -0.0]
    vals = np.array(vals, np.float64)
    with np.errstate(over="ignore"):
        ref = vals.astype(np.float16).view(np.uint16)
    got = np.array([oracle.f16_from_double(v) for v in vals], np.uint16)
    assert (got == ref).all(), vals[got != ref][:5]


def test_combine_f16_golden():
    c = _f16()["combine"]
    out = oracle.combine_f16(np.array(c["y"], np.uint16), np.array(c["w"], np.float32),
                             np.array(c["slot_idx"], np.int32))
    assert out.tolist() == c["out"], c["why"]


def test_combine_f16_one_hot_is_a_gather_and_round_trip_is_exact():
    g = np.random.default_rng(8)
    R, H, T, k = 40, 64, 10, 4
    y = (g.standard_normal((R, H)) * 100).astype(np.float16).view(np.uint16)
    slot = g.integers(-1, R, size=(T, k)).astype(np.int32)
    slot[:, 0] = g.integers(0, R, T)
    w = np.zeros((T, k), np.float32)
    w[:, 0] = 1.0
    assert (oracle.combine_f16(y, w, slot) == y[slot[:, 0]]).all()
    # the same row under weights that sum to 1 exactly: the row itself
    same = np.repeat(slot[:, :1], k, axis=1)
    w2 = np.tile(np.array([0.5, 0.25, 0.125, 0.125], np.float32), (T, 1))
    out = oracle.combine_f16(y, w2, same)
    assert ((out & 0x7FFF) == (y[slot[:, 0]] & 0x7FFF)).all()


def test_combine_f16_is_the_rounded_exact_sum():
    """Weights with few significant bits and values in a narrow binade range
    make every fp64 sum exact; numpy's float16 rounding of it is the reference."""
    g = np.random.default_rng(9)
    R, H, T, k = 30, 48, 12, 6
    y = (g.standard_normal((R, H)) * 8).astype(np.float16).view(np.uint16)
    slot = g.integers(-1, R, size=(T, k)).astype(np.int32)
    w = (g.integers(-64, 65, size=(T, k)) / 64.0).astype(np.float32)
    out = oracle.combine_f16(y, w, slot)
    yv = y.view(np.float16)
    for t in range(T):
        for c in range(H):
            acc = Fraction(0)
            for j in range(k):
                if slot[t, j] >= 0:
                    acc += Fraction(float(w[t, j])) * Fraction(float(yv[slot[t, j], c]))
            exact = float(acc)
            assert Fraction(exact) == acc
            assert out[t, c] == np.float16(exact).view(np.uint16) or (exact == 0 and out[t, c] == 0)


# --------------------------------------------------------------------------- MXFP8 combine
def test_combine_mxfp8_golden():
    """Hand-worked, H = 64 (two 32-channel blocks), k = 2.
    Row 0: codes 0x38 (1.0) except column 31, 0xB8 (-1.0); scale bytes 128, 129
    (2 and 4).  Row 1: codes 0x40 (2.0); bytes 126, 127 (0.5 and 1).
    Token 0 = 0.5 * row 0 + 0.25 * row 1:
      columns 0..30  0.5*1*2 + 0.25*2*0.5 = 1.25   (bf16 0x3FA0)
      column 31      0.5*-1*2 + 0.25*2*0.5 = -0.75 (0xBF40)
      columns 32..63 0.5*1*4 + 0.25*2*1 = 2.5      (0x4020)
    Token 1 = 1.0 * row 1, its second pair dropped: 1.0 (0x3F80), then 2.0 (0x4000).
    Token 2 has no valid pair: +0."""
    q = np.full((2, 64), 0x38, np.uint8)
    q[0, 31] = 0xB8
    q[1, :] = 0x40
    sc = np.array([[128, 129], [126, 127]], np.uint8)
    slot = np.array([[0, 1], [1, -1], [-1, -1]], np.int32)
    w = np.array([[0.5, 0.25], [1.0, 0.7], [0.3, 0.3]], np.float32)
    out = oracle.combine_mxfp8(q, sc, w, slot)
    want = np.zeros((3, 64), np.uint16)
    want[0, :31], want[0, 31], want[0, 32:] = 0x3FA0, 0xBF40, 0x4020
    want[1, :32], want[1, 32:] = 0x3F80, 0x4000
    assert (out == want).all(), [(r, c, hex(out[r, c]), hex(want[r, c])) for r, c in np.argwhere(out != want)[:4]]


def _mx_operands(g, R, H, lo=100, hi=155):
    q = g.integers(0, 256, (R, H)).astype(np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x31          # no NaN codes
    sc = g.integers(lo, hi, (R, H // 32)).astype(np.uint8)
    return q, sc


def test_dequant_mxfp8_extreme_scale_bytes():
    """The stand-in at the ends of the E8M0 range: bytes 0 and 1 (bf16
    subnormal products), 254 (overflow to infinity for codes of magnitude >= 2)
    and 255, NaN in E8M0, which turns its whole block into 0x7FC0 while the
    other blocks keep their values.  Reference: torch's float8_e4m3fn and
    float8_e8m0fnu decodes; every product here is exact in fp32."""
    codes = np.array([c for c in range(256) if (c & 0x7F) >= 0x38 and (c & 0x7F) != 0x7F], np.uint8)
    bytes_ = np.array([0, 1, 127, 254, 255], np.uint8)
    R, H = 2, 32 * bytes_.size
    q = np.resize(codes, (R, H)).astype(np.uint8)
    sc = np.tile(bytes_, (R, 1))
    y = oracle.dequant_mxfp8(q, sc)
    nan_block = np.repeat(sc == 255, 32, axis=1)
    assert (y[nan_block] == 0x7FC0).all()
    with np.errstate(over="ignore", invalid="ignore"):
        prod = _e4m3_values(q) * np.repeat(_e8m0_values(sc), 32, axis=1)
        prod = np.where(np.abs(prod) > 3.3895313892515355e38, np.copysign(np.inf, prod), prod)
        ref = (prod.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert (y[~nan_block] == ref[~nan_block]).all()


def test_combine_mxfp8_one_hot_is_the_dequantisation():
    g = np.random.default_rng(12)
    R, H, k = 40, 256, 4
    q, sc = _mx_operands(g, R, H)
    slot = np.full((R, k), -1, np.int32)
    slot[:, 2] = np.arange(R)
    w = g.random((R, k)).astype(np.float32)
    w[:, 2] = 1.0
    # equal up to the sign of zero: the sum starts at +0, so a -0 term (code 0x80) gives +0
    nz = lambda b: np.where(b == 0x8000, 0, b)
    assert (nz(oracle.combine_mxfp8(q, sc, w, slot)) == nz(oracle.dequant_mxfp8(q, sc))).all()


def test_combine_mxfp8_vs_float64_sum():
    """Within half a bf16 ulp of a float64 sum whose operands come from torch's
    float8_e4m3fn and float8_e8m0fnu decodes (independent of the oracle)."""
    g = np.random.default_rng(13)
    R, H, T, k = 300, 256, 64, 8
    q, sc = _mx_operands(g, R, H)
    slot = g.integers(-1, R, (T, k)).astype(np.int32)
    w = g.random((T, k)).astype(np.float32)
    out = unbf(oracle.combine_mxfp8(q, sc, w, slot)).astype(np.float64)
    vals = _e4m3_values(q) * np.repeat(_e8m0_values(sc), 32, 1)
    ref = np.zeros((T, H))
    for j in range(k):
        m = slot[:, j] >= 0
        ref[m] += w[m, j:j + 1].astype(np.float64) * vals[slot[m, j]]
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -126))) - 7)
    assert (np.abs(out - ref) <= 0.5 * ulp * (1 + 1e-9)).all()


def test_combine_mxfp8_extreme_scale_bytes():
    """One-hot weights over every E4M3 code of magnitude >= 1 and scale bytes
    from 0 (2^-127, whose products are bf16 subnormals) to 254 (2^127, whose
    products of magnitude >= 2 overflow to infinity): each output is the single
    product, exactly representable or infinite, compared with torch's
    float8_e4m3fn and float8_e8m0fnu decodes."""
    codes = np.array([c for c in range(256) if (c & 0x7F) >= 0x38 and (c & 0x7F) != 0x7F], np.uint8)
    bytes_ = np.array([0, 1, 2, 100, 127, 200, 253, 254], np.uint8)
    R, H = bytes_.size, 32 * ((codes.size + 31) // 32)
    q = np.resize(codes, (R, H)).astype(np.uint8)
    sc = np.repeat(bytes_[:, None], H // 32, 1)
    slot = np.arange(R, dtype=np.int32).reshape(R, 1)
    out = oracle.combine_mxfp8(q, sc, np.ones((R, 1), np.float32), slot)
    exact = _e4m3_values(q) * np.repeat(_e8m0_values(sc), 32, 1)
    with np.errstate(over="ignore"):
        want = np.where(np.abs(exact) > 3.3895313892515355e38, np.copysign(np.inf, exact), exact)
        want_bits = (want.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    finite = np.isfinite(want)
    assert (want.astype(np.float32)[finite].astype(np.float64) == want[finite]).all()
    assert (out == want_bits).all(), [(r, c, hex(out[r, c]), hex(want_bits[r, c]))
                                       for r, c in np.argwhere(out != want_bits)[:4]]


def test_combine_mxfp8_nan_scale_and_codes():
    """E8M0 byte 255 and E4M3 codes 0x7F / 0xFF are NaN; a NaN term makes its
    column NaN, and other columns are unaffected."""
    q = np.full((1, 64), 0x38, np.uint8)
    q[0, 40] = 0x7F
    sc = np.array([[255, 127]], np.uint8)
    out = unbf(oracle.combine_mxfp8(q, sc, np.ones((1, 1), np.float32), np.zeros((1, 1), np.int32)))
    assert np.isnan(out[0, :32]).all() and np.isnan(out[0, 40])
    assert (np.delete(out[0, 32:], 8) == 1.0).all()
