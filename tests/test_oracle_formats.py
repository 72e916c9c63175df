"""Pins for the oracle's number formats (CPU only).

The oracle's E4M3 encoder and bf16 rounding are checked against things other
than themselves: hand-worked values from the format definitions
(tests/golden/*.json), torch's independent float8_e4m3fn and bfloat16 casts
(exhaustively over every fp32 value the path can hand the FP8 encoder), and
exact rational arithmetic for rounding from binary64.
"""
import json
import os
from concurrent.futures import ThreadPoolExecutor
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _ev(expr):
    return float(eval(expr, {"__builtins__": {}}, {}))


# --------------------------------------------------------------------------- E4M3
def test_e4m3_golden_values():
    for expr, code, why in _load("e4m3_ocp_values.json")["cases"]:
        got = oracle.e4m3_encode(_ev(expr))
        assert got == int(code, 16), (expr, hex(got), code, why)


def test_e4m3_decode_table_is_the_format():
    # 254 finite codes (two NaN codes), symmetric, strictly increasing magnitudes,
    # largest finite 448, smallest subnormal 2**-9, smallest normal 2**-6.
    mags = [oracle.e4m3_decode(c) for c in range(0x7F)]
    assert all(b > a for a, b in zip(mags, mags[1:]))
    assert mags[0] == 0.0 and mags[1] == 2.0 ** -9 and mags[8] == 2.0 ** -6 and mags[126] == 448.0
    assert np.isnan(oracle.e4m3_decode(0x7F)) and np.isnan(oracle.e4m3_decode(0xFF))
    for c in range(0x7F):
        assert oracle.e4m3_decode(c | 0x80) == -mags[c]
    # every code decodes to a value the encoder maps back to the same code
    for c in list(range(0x7F)) + list(range(0x80, 0xFF)):
        assert oracle.e4m3_encode(oracle.e4m3_decode(c)) == c


def test_e4m3_matches_torch_decode():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = np.array([oracle.e4m3_decode(c) for c in range(256)])
    same = (ref == mine) | (np.isnan(ref) & np.isnan(mine))
    assert same.all()


def _torch_e4m3_bits(first, n):
    f = np.arange(first, first + n, dtype=np.uint64).astype(np.uint32).view(np.float32)
    return torch.from_numpy(f).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


@pytest.mark.parametrize("sign", [0, 1])
def test_e4m3_exhaustive_vs_torch(sign):
    """Every fp32 bit pattern with |v| <= 448 (the clamped range the encoder
    sees), one sign per case: ~1.14e9 values each, split over threads."""
    top = 0x43E00000  # 448.0
    base = 0x80000000 if sign else 0
    chunk = 1 << 24
    oracle.lib()

    def run(start):
        n = min(chunk, top + 1 - start)
        mine = oracle.e4m3_encode_bits(base + start, n)
        ref = _torch_e4m3_bits(base + start, n)
        bad = np.nonzero(mine != ref)[0]
        return [(hex(base + start + int(i)), int(mine[i]), int(ref[i])) for i in bad[:3]]

    with ThreadPoolExecutor(8) as ex:
        mismatches = [m for r in ex.map(run, range(0, top + 1, chunk)) for m in r]
    assert not mismatches, mismatches


# --------------------------------------------------------------------------- bf16
def test_bf16_golden_values():
    for expr, bits, why in _load("bf16_values.json")["cases"]:
        got = oracle.bf16_from_double(_ev(expr))
        assert got == int(bits, 16), (expr, hex(got), bits, why)


def test_bf16_matches_torch_on_float32_inputs():
    """torch rounds fp32 -> bf16 nearest-even; on fp32-exact inputs the oracle's
    rounding from binary64 must agree bit for bit (ties, subnormals, overflow)."""
    g = np.random.default_rng(7)
    u = g.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    # force many exact ties and near-ties: low 16 bits 0x8000, 0x7fff, 0x8001
    u[:30000] = (u[:30000] & 0xFFFF0000) | 0x8000
    u[30000:40000] = (u[30000:40000] & 0xFFFF0000) | 0x7FFF
    u[40000:50000] = (u[40000:50000] & 0xFFFF0000) | 0x8001
    f = u.view(np.float32)
    f = f[np.isfinite(f)]
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    mine = np.array([oracle.bf16_from_double(float(v)) for v in f], np.uint16)
    bad = np.nonzero(ref != mine)[0]
    assert bad.size == 0, [(hex(int(u)), hex(int(a)), hex(int(b)))
                           for u, a, b in zip(f[bad[:5]].view(np.uint32), mine[bad[:5]], ref[bad[:5]])]


def _bf16_exact_nearest(v: float) -> int:
    """Brute force with exact rationals: the bf16 value nearest to v among the
    two bf16 neighbours, ties to the even bit pattern."""
    x = Fraction(v)
    s = 0x8000 if (v < 0 or (v == 0 and np.signbit(v))) else 0
    a = abs(x)
    # enumerate candidates by bit pattern around the fp32 truncation of |v|
    base = int(np.array([abs(v)], np.float64).astype(np.float32).view(np.uint32)[0]) >> 16
    best = None
    for b in range(max(0, base - 2), min(0x7F80, base + 3) + 1):
        val = Fraction(0) if b == 0 else Fraction(
            float(np.array([b << 16], np.uint32).view(np.float32)[0])) if b < 0x7F80 else None
        if val is None:
            continue
        d = abs(val - a)
        if best is None or d < best[0] or (d == best[0] and b % 2 == 0):
            best = (d, b)
    return s | best[1]


def test_bf16_rounding_from_binary64_exact():
    g = np.random.default_rng(11)
    vals = list(g.standard_normal(3000) * np.exp2(g.integers(-130, 120, 3000)))
    # values that sit just off a bf16 midpoint by less than an fp32 ulp
    for m in range(1, 200):
        mid = (1 + (2 * m + 1) * 2.0 ** -8)
        vals += [mid, mid + 2.0 ** -40, mid - 2.0 ** -40]
    for v in vals:
        assert oracle.bf16_from_double(v) == _bf16_exact_nearest(v), v
