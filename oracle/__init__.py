"""CPU oracle for MoE dispatch / combine -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product (``combine_moe_layout_amd``)
never imports, loads or calls it, and it shares no code with the HIP library.

This module is a thin numpy <-> ctypes wrapper around ``ep_oracle.c``: plain,
single-threaded scalar loops written from the definitions on the pages (cited
in that file's header, with the readings R1..R21 it takes where the pages are
silent).  Every function here only marshals arrays; all arithmetic is in C.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ep_oracle.c")
_LIB = os.path.join(_HERE, "libep_oracle.so")

# Plain IEEE arithmetic: no fast-math, no contraction of a*b+c into one fma.
GCC_FLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared", "-std=c11"]


def build(force: bool = False) -> str:
    """Compile ep_oracle.c with gcc into libep_oracle.so (next to the source)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", *GCC_FLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load(path: str) -> ctypes.CDLL:
    L = ctypes.CDLL(path)
    i64, i32, u32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32, ctypes.c_void_p
    L.ep_oracle_bf16_to_double.restype = ctypes.c_double
    L.ep_oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
    L.ep_oracle_bf16_from_double.restype = ctypes.c_uint16
    L.ep_oracle_bf16_from_double.argtypes = [ctypes.c_double]
    L.ep_oracle_e4m3_decode.restype = ctypes.c_double
    L.ep_oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
    L.ep_oracle_e4m3_encode.restype = ctypes.c_uint8
    L.ep_oracle_e4m3_encode.argtypes = [ctypes.c_float]
    L.ep_oracle_e4m3_encode_array.argtypes = [vp, i64, vp]
    L.ep_oracle_e4m3_encode_bits.argtypes = [u32, i64, vp]
    L.ep_oracle_num_recv_rows.restype = i64
    L.ep_oracle_num_recv_rows.argtypes = [i64, i32, i32, i32]
    L.ep_oracle_layout.restype = ctypes.c_int
    L.ep_oracle_layout.argtypes = [vp, i64, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp]
    L.ep_oracle_dispatch_bf16.argtypes = [vp, i64, i32, i32, vp, vp]
    L.ep_oracle_quantize_token_fp8.argtypes = [vp, i32, vp, vp]
    L.ep_oracle_dispatch_fp8.argtypes = [vp, i64, i32, i32, vp, vp, vp]
    L.ep_oracle_scales_mn_major.argtypes = [vp, i64, i32, i32, vp]
    L.ep_oracle_combine_mxfp8.argtypes = [vp, vp, vp, vp, i64, i32, i32, vp]
    L.ep_oracle_combine_mxfp8_tokens.argtypes = [vp, vp, vp, vp, i32, i32, vp, i64, vp]
    L.ep_oracle_dequant_fp8.argtypes = [vp, vp, i64, i32, vp]
    L.ep_oracle_combine.argtypes = [vp, vp, vp, i64, i32, i32, vp]
    L.ep_oracle_combine_tokens.argtypes = [vp, vp, vp, i32, i32, vp, i64, vp]
    L.ep_oracle_quantize_token_fp8_pow2.argtypes = [vp, i32, vp, vp]
    L.ep_oracle_dispatch_fp8_pow2.argtypes = [vp, i64, i32, i32, vp, vp, vp]
    L.ep_oracle_combine_fp8.argtypes = [vp, vp, vp, vp, i64, i32, i32, vp]
    L.ep_oracle_combine_fp8_tokens.argtypes = [vp, vp, vp, vp, i32, i32, vp, i64, vp]
    L.ep_oracle_group_layout.restype = ctypes.c_int
    L.ep_oracle_group_layout.argtypes = [vp, vp, i64, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.ep_oracle_combine_groups.argtypes = [vp, vp, i64, i32, i32, vp]
    L.ep_oracle_combine_groups_tokens.argtypes = [vp, vp, i32, i32, vp, i64, vp]
    L.ep_oracle_quantize_token_mxfp8.argtypes = [vp, i32, vp, vp]
    L.ep_oracle_dispatch_mxfp8.argtypes = [vp, i64, i32, i32, vp, vp, vp]
    L.ep_oracle_dequant_mxfp8.argtypes = [vp, vp, i64, i32, vp]
    L.ep_oracle_f16_to_double.restype = ctypes.c_double
    L.ep_oracle_f16_to_double.argtypes = [ctypes.c_uint16]
    L.ep_oracle_f16_from_double.restype = ctypes.c_uint16
    L.ep_oracle_f16_from_double.argtypes = [ctypes.c_double]
    L.ep_oracle_combine_f16.argtypes = [vp, vp, vp, i64, i32, i32, vp]
    L.ep_oracle_combine_f16_tokens.argtypes = [vp, vp, vp, i32, i32, vp, i64, vp]
    return L


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        build()
        _lib = _load(_LIB)
    return _lib


@contextlib.contextmanager
def use_library(path: str):
    """Temporarily route every wrapper through another build of the oracle
    (used by the test that checks the pins catch planted mistakes)."""
    global _lib
    saved = lib()
    _lib = _load(path)
    try:
        yield
    finally:
        _lib = saved


def _p(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


# ----------------------------------------------------------------------------- scalars
def bf16_to_float(bits) -> float:
    return lib().ep_oracle_bf16_to_double(int(bits) & 0xFFFF)


def bf16_from_double(v: float) -> int:
    return int(lib().ep_oracle_bf16_from_double(float(v)))


def e4m3_decode(code: int) -> float:
    return lib().ep_oracle_e4m3_decode(int(code) & 0xFF)


def e4m3_encode(v: float) -> int:
    return int(lib().ep_oracle_e4m3_encode(float(v)))


def e4m3_encode_array(v: np.ndarray) -> np.ndarray:
    v = _c(v, np.float32).reshape(-1)
    out = np.empty(v.size, np.uint8)
    lib().ep_oracle_e4m3_encode_array(_p(v), v.size, _p(out))
    return out


def e4m3_encode_bits(first: int, n: int, out: np.ndarray | None = None) -> np.ndarray:
    if out is None:
        out = np.empty(n, np.uint8)
    lib().ep_oracle_e4m3_encode_bits(ctypes.c_uint32(first), n, _p(out))
    return out


# ----------------------------------------------------------------------------- layout
def num_recv_rows(T: int, k: int, E: int, cap: int) -> int:
    return int(lib().ep_oracle_num_recv_rows(T, k, E, cap))


def layout(topk_idx: np.ndarray, E: int, G: int = 1, cap: int = 0, want_recv_src: bool = True):
    """Returns a dict: num_tokens_per_expert [E], expert_offsets [E+1],
    num_tokens_per_group [G], slot_idx [T,k], recv_src [R] (or None), error_flags."""
    topk_idx = _c(topk_idx, np.int64)
    T, k = topk_idx.shape
    R = num_recv_rows(T, k, E, cap)
    cnt = np.zeros(E, np.int32)
    off = np.zeros(E + 1, np.int32)
    grp = np.zeros(G, np.int32)
    slot = np.empty((T, k), np.int32)
    src = np.full(R, -1, np.int32) if want_recv_src else None
    flags = np.zeros(1, np.int32)
    rc = lib().ep_oracle_layout(_p(topk_idx) if T else None, T, k, E, G, cap, _p(cnt), _p(off),
                                _p(grp), _p(slot) if T else None,
                                _p(src) if src is not None and R > 0 else None, _p(flags))
    if rc != 0:
        raise ValueError("oracle layout rejected its arguments (status %d)" % rc)
    return dict(num_tokens_per_expert=cnt, expert_offsets=off, num_tokens_per_group=grp,
                slot_idx=slot, recv_src=src, error_flags=int(flags[0]), num_recv_rows=R)


# ----------------------------------------------------------------------------- dispatch
def dispatch_bf16(x_bits: np.ndarray, slot_idx: np.ndarray, R: int) -> np.ndarray:
    """x_bits: uint16 [T,H] bf16 bit patterns.  Rows no slot addresses stay 0."""
    x_bits = _c(x_bits, np.uint16)
    slot_idx = _c(slot_idx, np.int32)
    T, H = x_bits.shape
    k = slot_idx.shape[1]
    recv = np.zeros((R, H), np.uint16)
    lib().ep_oracle_dispatch_bf16(_p(x_bits), T, k, H, _p(slot_idx), _p(recv))
    return recv


def quantize_token_fp8(x_row_bits: np.ndarray):
    x_row_bits = _c(x_row_bits, np.uint16).reshape(-1)
    H = x_row_bits.size
    q = np.empty(H, np.uint8)
    s = np.empty(H // 128, np.float32)
    lib().ep_oracle_quantize_token_fp8(_p(x_row_bits), H, _p(q), _p(s))
    return q, s


def dispatch_fp8(x_bits: np.ndarray, slot_idx: np.ndarray, R: int):
    """Returns (recv_q uint8 [R,H], recv_scales float32 [R,H/128]); rows no slot
    addresses stay 0."""
    x_bits = _c(x_bits, np.uint16)
    slot_idx = _c(slot_idx, np.int32)
    T, H = x_bits.shape
    k = slot_idx.shape[1]
    q = np.zeros((R, H), np.uint8)
    s = np.zeros((R, H // 128), np.float32)
    lib().ep_oracle_dispatch_fp8(_p(x_bits), T, k, H, _p(slot_idx), _p(q), _p(s))
    return q, s


def dispatch_fp8_into(x_bits: np.ndarray, slot_idx: np.ndarray, q: np.ndarray,
                      s: np.ndarray) -> None:
    """dispatch_fp8 of the tokens in x_bits (a contiguous range of rows) with
    their slot rows, written into the caller's receive arrays q [R,H] and
    s [R,H/128].  Different token ranges write disjoint receive rows, so
    ranges may run on separate threads (the C call releases the GIL)."""
    assert x_bits.flags.c_contiguous and slot_idx.flags.c_contiguous
    assert x_bits.dtype == np.uint16 and slot_idx.dtype == np.int32
    assert q.flags.c_contiguous and s.flags.c_contiguous and q.dtype == np.uint8 and s.dtype == np.float32
    T, H = x_bits.shape
    assert slot_idx.shape[0] == T and q.shape[1] == H and s.shape == (q.shape[0], H // 128)
    lib().ep_oracle_dispatch_fp8(_p(x_bits), T, slot_idx.shape[1], H, _p(slot_idx), _p(q), _p(s))


def dequant_fp8(q: np.ndarray, scales: np.ndarray) -> np.ndarray:
    q = _c(q, np.uint8)
    scales = _c(scales, np.float32)
    R, H = q.shape
    y = np.empty((R, H), np.uint16)
    lib().ep_oracle_dequant_fp8(_p(q), _p(scales), R, H, _p(y))
    return y


# ----------------------------------------------------------------------------- combine
def combine(y_bits: np.ndarray, w: np.ndarray, slot_idx: np.ndarray) -> np.ndarray:
    y_bits = _c(y_bits, np.uint16)
    w = _c(w, np.float32)
    slot_idx = _c(slot_idx, np.int32)
    T, k = slot_idx.shape
    H = y_bits.shape[1]
    out = np.empty((T, H), np.uint16)
    lib().ep_oracle_combine(_p(y_bits), _p(w), _p(slot_idx), T, k, H, _p(out))
    return out


def combine_into(y_bits: np.ndarray, w: np.ndarray, slot_idx: np.ndarray, out: np.ndarray) -> None:
    """combine of the tokens whose weight and slot rows are given (a
    contiguous range), written into out (the same range of output rows); the
    C call releases the GIL, so ranges may run on separate threads."""
    for a, dt in ((y_bits, np.uint16), (w, np.float32), (slot_idx, np.int32), (out, np.uint16)):
        assert a.flags.c_contiguous and a.dtype == dt
    T, k = slot_idx.shape
    H = y_bits.shape[1]
    assert w.shape == (T, k) and out.shape == (T, H)
    lib().ep_oracle_combine(_p(y_bits), _p(w), _p(slot_idx), T, k, H, _p(out))


def combine_tokens(y_bits: np.ndarray, w: np.ndarray, slot_idx: np.ndarray, tokens) -> np.ndarray:
    y_bits = _c(y_bits, np.uint16)
    w = _c(w, np.float32)
    slot_idx = _c(slot_idx, np.int32)
    tokens = _c(tokens, np.int64).reshape(-1)
    k = slot_idx.shape[1]
    H = y_bits.shape[1]
    out = np.empty((tokens.size, H), np.uint16)
    lib().ep_oracle_combine_tokens(_p(y_bits), _p(w), _p(slot_idx), k, H, _p(tokens),
                                   tokens.size, _p(out))
    return out


def chain_fp8_tokens(x_bits: np.ndarray, w: np.ndarray, slot_idx: np.ndarray, tokens) -> np.ndarray:
    """Full path for single tokens with identity experts and FP8 dispatch:
    every valid receive row of token t holds t's codes and scales, so the
    expert output at each of t's slots is dequant(quantize(x_t)); combine sums
    those with t's weights.  Built only from the oracle's own functions."""
    tokens = np.asarray(tokens, np.int64).reshape(-1)
    H = x_bits.shape[1]
    k = slot_idx.shape[1]
    out = np.empty((tokens.size, H), np.uint16)
    for i, t in enumerate(tokens):
        q, s = quantize_token_fp8(x_bits[t])
        yrow = dequant_fp8(q.reshape(1, H), s.reshape(1, -1))
        local_slot = np.where(np.asarray(slot_idx[t]) >= 0, 0, -1).astype(np.int32).reshape(1, k)
        out[i] = combine(yrow, np.asarray(w[t], np.float32).reshape(1, k), local_slot)[0]
    return out


def chain_bf16_tokens(x_bits: np.ndarray, w: np.ndarray, slot_idx: np.ndarray, tokens) -> np.ndarray:
    """Full path for single tokens with identity experts and bf16 dispatch."""
    tokens = np.asarray(tokens, np.int64).reshape(-1)
    H = x_bits.shape[1]
    k = slot_idx.shape[1]
    out = np.empty((tokens.size, H), np.uint16)
    for i, t in enumerate(tokens):
        yrow = np.ascontiguousarray(x_bits[t], np.uint16).reshape(1, H)
        local_slot = np.where(np.asarray(slot_idx[t]) >= 0, 0, -1).astype(np.int32).reshape(1, k)
        out[i] = combine(yrow, np.asarray(w[t], np.float32).reshape(1, k), local_slot)[0]
    return out


# ----------------------------------------------------------------------------- variants
def quantize_token_fp8_pow2(x_row_bits: np.ndarray):
    """Power-of-two scales (reading R13)."""
    x_row_bits = _c(x_row_bits, np.uint16).reshape(-1)
    H = x_row_bits.size
    q = np.empty(H, np.uint8)
    s = np.empty(H // 128, np.float32)
    lib().ep_oracle_quantize_token_fp8_pow2(_p(x_row_bits), H, _p(q), _p(s))
    return q, s


def dispatch_fp8_pow2(x_bits: np.ndarray, slot_idx: np.ndarray, R: int):
    x_bits = _c(x_bits, np.uint16)
    slot_idx = _c(slot_idx, np.int32)
    T, H = x_bits.shape
    k = slot_idx.shape[1]
    q = np.zeros((R, H), np.uint8)
    s = np.zeros((R, H // 128), np.float32)
    lib().ep_oracle_dispatch_fp8_pow2(_p(x_bits), T, k, H, _p(slot_idx), _p(q), _p(s))
    return q, s


def combine_fp8(q: np.ndarray, scales: np.ndarray, w: np.ndarray, slot_idx: np.ndarray) -> np.ndarray:
    """Combine of FP8 expert outputs (reading R14)."""
    q = _c(q, np.uint8)
    scales = _c(scales, np.float32)
    w = _c(w, np.float32)
    slot_idx = _c(slot_idx, np.int32)
    T, k = slot_idx.shape
    H = q.shape[1]
    out = np.empty((T, H), np.uint16)
    lib().ep_oracle_combine_fp8(_p(q), _p(scales), _p(w), _p(slot_idx), T, k, H, _p(out))
    return out


def combine_fp8_tokens(q, scales, w, slot_idx, tokens) -> np.ndarray:
    q = _c(q, np.uint8)
    scales = _c(scales, np.float32)
    w = _c(w, np.float32)
    slot_idx = _c(slot_idx, np.int32)
    tokens = _c(tokens, np.int64).reshape(-1)
    k = slot_idx.shape[1]
    H = q.shape[1]
    out = np.empty((tokens.size, H), np.uint16)
    lib().ep_oracle_combine_fp8_tokens(_p(q), _p(scales), _p(w), _p(slot_idx), k, H, _p(tokens),
                                       tokens.size, _p(out))
    return out


# ----------------------------------------------------------------------------- dedup variant
def group_layout(topk_idx: np.ndarray, topk_weights: np.ndarray | None, E: int, G: int):
    """Per-group dedup layout (readings R15, R16).  Returns a dict:
    group_idx [T,kg], num_tokens_per_group [G], group_offsets [G+1],
    group_slot [T,kg], recv_token [T*kg] (-1 in unused rows),
    recv_topk_idx [T*kg,k] (-1 in unused rows), recv_topk_weights [T*kg,k]
    (0 in unused rows, or None without weights), is_token_in_group [T,G]
    (uint8, 1 where the token reaches the group), error_flags, kg, rows_used."""
    topk_idx = _c(topk_idx, np.int64)
    T, k = topk_idx.shape
    kg = min(k, G)
    R = T * kg
    gidx = np.empty((T, kg), np.int32)
    cnt = np.zeros(G, np.int32)
    off = np.zeros(G + 1, np.int32)
    slot = np.empty((T, kg), np.int32)
    tok = np.full(R, -1, np.int32)
    ridx = np.full((R, k), -1, np.int64)
    rw = None
    if topk_weights is not None:
        topk_weights = _c(topk_weights, np.float32)
        rw = np.zeros((R, k), np.float32)
    flags = np.zeros(1, np.int32)
    member = np.zeros((T, G), np.uint8)
    has = T > 0
    rc = lib().ep_oracle_group_layout(_p(topk_idx) if has else None,
                                      _p(topk_weights) if rw is not None and has else None,
                                      T, k, E, G, _p(gidx) if has else None, _p(cnt), _p(off),
                                      _p(slot) if has else None, _p(tok) if R else None,
                                      _p(ridx) if R else None, _p(rw) if rw is not None and R else None,
                                      _p(member) if has else None, _p(flags))
    if rc != 0:
        raise ValueError("oracle group layout rejected its arguments (status %d)" % rc)
    return dict(group_idx=gidx, num_tokens_per_group=cnt, group_offsets=off, group_slot=slot,
                recv_token=tok, recv_topk_idx=ridx, recv_topk_weights=rw, is_token_in_group=member,
                error_flags=int(flags[0]), kg=kg, rows_used=int(off[G]))


def combine_groups(z_bits: np.ndarray, group_slot: np.ndarray) -> np.ndarray:
    """Group combine of the dedup variant (reading R17): unit-weight sum of a
    token's group rows."""
    z_bits = _c(z_bits, np.uint16)
    group_slot = _c(group_slot, np.int32)
    T, kg = group_slot.shape
    H = z_bits.shape[1]
    out = np.empty((T, H), np.uint16)
    lib().ep_oracle_combine_groups(_p(z_bits), _p(group_slot), T, kg, H, _p(out))
    return out


def combine_groups_tokens(z_bits: np.ndarray, group_slot: np.ndarray, tokens) -> np.ndarray:
    z_bits = _c(z_bits, np.uint16)
    group_slot = _c(group_slot, np.int32)
    tokens = _c(tokens, np.int64).reshape(-1)
    kg = group_slot.shape[1]
    H = z_bits.shape[1]
    out = np.empty((tokens.size, H), np.uint16)
    lib().ep_oracle_combine_groups_tokens(_p(z_bits), _p(group_slot), kg, H, _p(tokens),
                                          tokens.size, _p(out))
    return out


# ----------------------------------------------------------------------------- MXFP8 and FP16 variants
def quantize_token_mxfp8(x_row_bits: np.ndarray):
    """MXFP8 (reading R18): codes [H] and E8M0 scale bytes [H/32]."""
    x_row_bits = _c(x_row_bits, np.uint16).reshape(-1)
    H = x_row_bits.size
    q = np.empty(H, np.uint8)
    s = np.empty(H // 32, np.uint8)
    lib().ep_oracle_quantize_token_mxfp8(_p(x_row_bits), H, _p(q), _p(s))
    return q, s


def dispatch_mxfp8(x_bits: np.ndarray, slot_idx: np.ndarray, R: int):
    x_bits = _c(x_bits, np.uint16)
    slot_idx = _c(slot_idx, np.int32)
    T, H = x_bits.shape
    k = slot_idx.shape[1]
    q = np.zeros((R, H), np.uint8)
    s = np.zeros((R, H // 32), np.uint8)
    lib().ep_oracle_dispatch_mxfp8(_p(x_bits), T, k, H, _p(slot_idx), _p(q), _p(s))
    return q, s


def dequant_mxfp8(q: np.ndarray, scales: np.ndarray) -> np.ndarray:
    q = _c(q, np.uint8)
    scales = _c(scales, np.uint8)
    R, H = q.shape
    y = np.empty((R, H), np.uint16)
    lib().ep_oracle_dequant_mxfp8(_p(q), _p(scales), R, H, _p(y))
    return y


def f16_to_double(bits: int) -> float:
    return float(lib().ep_oracle_f16_to_double(int(bits)))


def f16_from_double(v: float) -> int:
    return int(lib().ep_oracle_f16_from_double(float(v)))


def combine_f16(y_bits: np.ndarray, w: np.ndarray, slot_idx: np.ndarray) -> np.ndarray:
    """fp16 combine (reading R19): y and out are binary16 bit patterns."""
    y_bits = _c(y_bits, np.uint16)
    w = _c(w, np.float32)
    slot_idx = _c(slot_idx, np.int32)
    T, k = slot_idx.shape
    H = y_bits.shape[1]
    out = np.empty((T, H), np.uint16)
    lib().ep_oracle_combine_f16(_p(y_bits), _p(w), _p(slot_idx), T, k, H, _p(out))
    return out


def combine_f16_tokens(y_bits: np.ndarray, w: np.ndarray, slot_idx: np.ndarray, tokens) -> np.ndarray:
    y_bits = _c(y_bits, np.uint16)
    w = _c(w, np.float32)
    slot_idx = _c(slot_idx, np.int32)
    tokens = _c(tokens, np.int64).reshape(-1)
    k = slot_idx.shape[1]
    H = y_bits.shape[1]
    out = np.empty((tokens.size, H), np.uint16)
    lib().ep_oracle_combine_f16_tokens(_p(y_bits), _p(w), _p(slot_idx), k, H, _p(tokens),
                                       tokens.size, _p(out))
    return out


def scales_mn_major(scales: np.ndarray) -> np.ndarray:
    """R20: row-major scales [R, n] (fp32 or E8M0 bytes) -> MN-major [n, R],
    entry c of row r at c * R + r."""
    src = np.ascontiguousarray(scales)
    rows, n = src.shape
    out = np.empty((n, rows), dtype=src.dtype)
    lib().ep_oracle_scales_mn_major(_p(src), rows, n, src.dtype.itemsize, _p(out))
    return out


def combine_mxfp8(q: np.ndarray, scales: np.ndarray, w: np.ndarray, slot_idx: np.ndarray) -> np.ndarray:
    """Combine of MXFP8 expert outputs (reading R21): codes [R, H], E8M0 bytes [R, H/32]."""
    q = _c(q, np.uint8)
    scales = _c(scales, np.uint8)
    w = _c(w, np.float32)
    slot_idx = _c(slot_idx, np.int32)
    T, k = slot_idx.shape
    H = q.shape[1]
    out = np.empty((T, H), np.uint16)
    lib().ep_oracle_combine_mxfp8(_p(q), _p(scales), _p(w), _p(slot_idx), T, k, H, _p(out))
    return out


def combine_mxfp8_tokens(q, scales, w, slot_idx, tokens) -> np.ndarray:
    q = _c(q, np.uint8)
    scales = _c(scales, np.uint8)
    w = _c(w, np.float32)
    slot_idx = _c(slot_idx, np.int32)
    tokens = _c(tokens, np.int64).reshape(-1)
    k = slot_idx.shape[1]
    H = q.shape[1]
    out = np.empty((tokens.size, H), np.uint16)
    lib().ep_oracle_combine_mxfp8_tokens(_p(q), _p(scales), _p(w), _p(slot_idx), k, H, _p(tokens),
                                         tokens.size, _p(out))
    return out
