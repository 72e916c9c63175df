"""ctypes binding of libep.so: the same entry points as include/ep.h.

Argument marshalling only: tensors become device pointers, torch's current
stream becomes the HIP stream, and a non-zero status becomes an exception.
Every step of the path runs in the HIP kernels; there is no fallback -- if the
library is missing or the tensors are not on the GPU, calls raise.
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libep.so")

EP_OK = 0
EP_BF16 = 0
EP_FP8_E4M3 = 1
EP_FP8_E4M3_POW2 = 2
EP_MXFP8_E4M3 = 3
EP_F16 = 4
EP_SCALES_MN_MAJOR = 0x100   # OR-ed into an FP8 dtype: scales stored transposed
EP_READ_X_AHEAD = 0x200      # OR-ed into ep_layout_dispatch's dtype: x read into the MALL during the layout
_FP8_DTYPES = (EP_FP8_E4M3, EP_FP8_E4M3_POW2, EP_MXFP8_E4M3)
EP_FLAG_BAD_EXPERT = 1
EP_FLAG_OVERFLOW = 2
EP_MAX_EXPERTS = 1024
EP_MAX_TOPK = 64
EP_MAX_HIDDEN = 65536
EP_NOALLOC_SCRATCH_BYTES = 4 << 20


class EpError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__("%s failed with status %d: %s" % (fn, status, text))
        self.status = status


class ep_layout_t(ctypes.Structure):
    _fields_ = [
        ("num_tokens", ctypes.c_int64),
        ("num_recv_rows", ctypes.c_int64),
        ("num_topk", ctypes.c_int32),
        ("num_experts", ctypes.c_int32),
        ("num_groups", ctypes.c_int32),
        ("capacity", ctypes.c_int32),
        ("num_tokens_per_expert", ctypes.c_void_p),
        ("expert_offsets", ctypes.c_void_p),
        ("num_tokens_per_group", ctypes.c_void_p),
        ("slot_idx", ctypes.c_void_p),
        ("recv_src", ctypes.c_void_p),
        ("error_flags", ctypes.c_void_p),
    ]


# name -> (restype, argtypes), mirroring include/ep.h
_i64, _i32, _u32, _vp, _sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_size_t
_LP = ctypes.POINTER(ep_layout_t)
SIGNATURES = {
    "ep_layout_init": (ctypes.c_int, [_LP, _i64, _i32, _i32, _i32, _i32]),
    "ep_num_recv_rows": (_i64, [_i64, _i32, _i32, _i32]),
    "ep_layout_workspace_bytes": (_sz, [_i64, _i32, _i32]),
    "ep_get_layout": (ctypes.c_int, [_vp, _LP, _vp, _sz, _vp]),
    "ep_get_layout_noalloc": (ctypes.c_int, [_vp, _LP, _vp]),
    "ep_dispatch": (ctypes.c_int, [_vp, _LP, _i32, _i32, _vp, _vp, _vp]),
    "ep_layout_dispatch": (ctypes.c_int, [_vp, _LP, _vp, _sz, _vp, _i32, _i32, _vp, _vp, _vp]),
    "ep_scales_to_mn_major": (ctypes.c_int, [_vp, _i64, _i32, _i32, _vp, _vp]),
    "ep_combine": (ctypes.c_int, [_vp, _vp, _LP, _i32, _vp, _vp]),
    "ep_combine_fp8": (ctypes.c_int, [_vp, _vp, _vp, _LP, _i32, _vp, _vp]),
    "ep_combine_f16": (ctypes.c_int, [_vp, _vp, _LP, _i32, _vp, _vp]),
    "ep_combine_mxfp8": (ctypes.c_int, [_vp, _vp, _vp, _LP, _i32, _vp, _vp]),
    "ep_dequant_mxfp8": (ctypes.c_int, [_vp, _vp, _i64, _i32, _vp, _vp]),
    "ep_group_layout_init": (ctypes.c_int, [_LP, _i64, _i32, _i32]),
    "ep_group_layout_workspace_bytes": (_sz, [_i64, _i32, _i32]),
    "ep_get_group_layout": (ctypes.c_int, [_vp, _vp, _i32, _i32, _LP, _vp, _vp, _vp, _vp, _sz, _vp]),
    "ep_combine_groups": (ctypes.c_int, [_vp, _LP, _i32, _vp, _vp]),
    "ep_dequant_fp8": (ctypes.c_int, [_vp, _vp, _i64, _i32, _vp, _vp]),
    "ep_cast_e4m3_bits": (ctypes.c_int, [_u32, _i64, _i32, _vp, _vp]),
    "ep_copy": (ctypes.c_int, [_vp, _vp, _sz, _vp]),
    "ep_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "ep_version": (ctypes.c_char_p, []),
}

_lib = None


def library_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """The loaded libep.so.  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError("libep.so is not built (%s); run `python -m "
                               "combine_moe_layout_amd.build`" % _LIB_PATH)
        L = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(fn: str, status: int) -> None:
    if status != EP_OK:
        raise EpError(fn, status, lib().ep_status_string(status).decode())


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _ptr(t: torch.Tensor | None, name: str, dtype=None) -> int | None:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    return t.data_ptr()


class EpLayout:
    """Device arrays of one routing layout plus the ep_layout_t that points at
    them (the handle passed from ep_get_layout to ep_dispatch / ep_combine)."""

    def __init__(self, num_tokens: int, num_topk: int, num_experts: int, num_groups: int = 1,
                 capacity: int = 0, with_recv_src: bool = False, device=None):
        self.struct = ep_layout_t()
        _check("ep_layout_init", lib().ep_layout_init(ctypes.byref(self.struct), num_tokens,
                                                      num_topk, num_experts, num_groups, capacity))
        self._alloc(with_recv_src, device,
                    lib().ep_layout_workspace_bytes(num_tokens, num_topk, num_experts))

    def _alloc(self, with_recv_src: bool, device, workspace_bytes: int) -> None:
        """Device arrays for the sizes in self.struct, and the struct's pointers to them."""
        s = self.struct
        dev = torch.device("cuda") if device is None else torch.device(device)
        i32 = dict(dtype=torch.int32, device=dev)
        self.num_tokens_per_expert = torch.empty(s.num_experts, **i32)
        self.expert_offsets = torch.empty(s.num_experts + 1, **i32)
        self.num_tokens_per_group = torch.empty(s.num_groups, **i32)
        self.slot_idx = torch.empty((s.num_tokens, s.num_topk), **i32)
        self.recv_src = torch.empty(s.num_recv_rows, **i32) if with_recv_src else None
        self.error_flags = torch.empty(1, **i32)
        s.num_tokens_per_expert = self.num_tokens_per_expert.data_ptr()
        s.expert_offsets = self.expert_offsets.data_ptr()
        s.num_tokens_per_group = self.num_tokens_per_group.data_ptr()
        s.slot_idx = self.slot_idx.data_ptr() if s.num_tokens > 0 else None
        s.recv_src = self.recv_src.data_ptr() if with_recv_src and self.recv_src.numel() else None
        s.error_flags = self.error_flags.data_ptr()
        self.workspace = torch.empty(workspace_bytes, dtype=torch.uint8, device=dev)

    @property
    def num_tokens(self) -> int:
        return self.struct.num_tokens

    @property
    def num_topk(self) -> int:
        return self.struct.num_topk

    @property
    def num_experts(self) -> int:
        return self.struct.num_experts

    @property
    def num_recv_rows(self) -> int:
        return self.struct.num_recv_rows


class EpGroupLayout(EpLayout):
    """The per-group dedup layout: an EpLayout whose "experts" are the G groups,
    with kg = min(k, G) entries per token (ep_group_layout_init).  It is
    accepted wherever an EpLayout is, so ep_dispatch sends to the groups."""

    def __init__(self, num_tokens: int, num_topk: int, num_experts: int, num_groups: int,
                 with_recv_src: bool = False, device=None):
        self.struct = ep_layout_t()
        _check("ep_group_layout_init", lib().ep_group_layout_init(
            ctypes.byref(self.struct), num_tokens, num_topk, num_groups))
        self.source_topk = num_topk
        self.source_experts = num_experts
        self._alloc(with_recv_src, device,
                    lib().ep_group_layout_workspace_bytes(num_tokens, num_topk, num_groups))


# ----------------------------------------------------------------------------- entry points
def ep_num_recv_rows(num_tokens: int, num_topk: int, num_experts: int, capacity: int = 0) -> int:
    return int(lib().ep_num_recv_rows(num_tokens, num_topk, num_experts, capacity))


def ep_layout_workspace_bytes(num_tokens: int, num_topk: int, num_experts: int) -> int:
    return int(lib().ep_layout_workspace_bytes(num_tokens, num_topk, num_experts))


def ep_get_layout(topk_idx: torch.Tensor, layout: EpLayout, stream=None) -> EpLayout:
    """topk_idx: int64 [T, k] on the GPU.  Fills layout's arrays."""
    if tuple(topk_idx.shape) != (layout.num_tokens, layout.num_topk):
        raise ValueError("topk_idx shape %s does not match the layout" % (tuple(topk_idx.shape),))
    _check("ep_get_layout", lib().ep_get_layout(
        _ptr(topk_idx, "topk_idx", torch.int64) if topk_idx.numel() else None,
        ctypes.byref(layout.struct), layout.workspace.data_ptr(), layout.workspace.numel(),
        _stream(stream)))
    return layout


def ep_get_layout_noalloc(topk_idx: torch.Tensor, layout: EpLayout, stream=None) -> EpLayout:
    """ep_get_layout with the library's own fixed per-GPU workspace instead of
    layout.workspace (for callers that cannot allocate at call time)."""
    if tuple(topk_idx.shape) != (layout.num_tokens, layout.num_topk):
        raise ValueError("topk_idx shape %s does not match the layout" % (tuple(topk_idx.shape),))
    _check("ep_get_layout_noalloc", lib().ep_get_layout_noalloc(
        _ptr(topk_idx, "topk_idx", torch.int64) if topk_idx.numel() else None,
        ctypes.byref(layout.struct), _stream(stream)))
    return layout


def _dispatch_types(recv_dtype: int):
    """(x dtype, recv_x dtype, recv_scales dtype) of a receive dtype (with or
    without EP_SCALES_MN_MAJOR)."""
    recv_dtype &= ~(EP_SCALES_MN_MAJOR | EP_READ_X_AHEAD)
    if recv_dtype == EP_F16:
        return torch.float16, torch.float16, None
    if recv_dtype == EP_MXFP8_E4M3:
        return torch.bfloat16, torch.uint8, torch.uint8
    if recv_dtype in _FP8_DTYPES:
        return torch.bfloat16, torch.uint8, torch.float32
    return torch.bfloat16, torch.bfloat16, None


def _check_scales(recv_dtype: int, recv_scales, R: int, H: int) -> None:
    """Every FP8 scale layout holds H/128 four-byte words per receive row."""
    if (recv_dtype & ~(EP_SCALES_MN_MAJOR | EP_READ_X_AHEAD)) in _FP8_DTYPES and recv_scales is not None:
        if recv_scales.numel() * recv_scales.element_size() != R * (H // 128) * 4:
            raise ValueError("recv_scales does not hold %d rows of %d channels' scales" % (R, H))


def ep_dispatch(x: torch.Tensor, layout: EpLayout, recv_dtype: int, recv_x: torch.Tensor,
                recv_scales: torch.Tensor | None = None, stream=None) -> None:
    """x bf16 [T, H] -> recv_x: bf16 [R, H]; uint8 [R, H] FP8 codes with
    recv_scales fp32 [R, H/128] (EP_FP8_E4M3, EP_FP8_E4M3_POW2) or uint8
    [R, H/32] E8M0 bytes (EP_MXFP8_E4M3), or their transposes [H/128, R] and
    [H/32, R] with EP_SCALES_MN_MAJOR.  EP_F16: x and recv_x fp16."""
    T, H = layout.num_tokens, x.shape[-1]
    if tuple(x.shape) != (T, H) or tuple(recv_x.shape) != (layout.num_recv_rows, H):
        raise ValueError("dispatch buffers do not match the layout")
    _check_scales(recv_dtype, recv_scales, layout.num_recv_rows, H)
    xt, rt, st = _dispatch_types(recv_dtype)
    _check("ep_dispatch", lib().ep_dispatch(
        _ptr(x, "x", xt), ctypes.byref(layout.struct), H, recv_dtype,
        _ptr(recv_x, "recv_x", rt), _ptr(recv_scales, "recv_scales", st),
        _stream(stream)))


def ep_layout_dispatch(topk_idx: torch.Tensor, layout: EpLayout, x: torch.Tensor, recv_dtype: int,
                       recv_x: torch.Tensor, recv_scales: torch.Tensor | None = None,
                       stream=None) -> EpLayout:
    """ep_get_layout followed by ep_dispatch; one launch for decode-sized batches."""
    T, H = layout.num_tokens, x.shape[-1]
    if tuple(topk_idx.shape) != (T, layout.num_topk):
        raise ValueError("topk_idx shape %s does not match the layout" % (tuple(topk_idx.shape),))
    if tuple(x.shape) != (T, H) or tuple(recv_x.shape) != (layout.num_recv_rows, H):
        raise ValueError("dispatch buffers do not match the layout")
    _check_scales(recv_dtype, recv_scales, layout.num_recv_rows, H)
    xt, rt, st = _dispatch_types(recv_dtype)
    _check("ep_layout_dispatch", lib().ep_layout_dispatch(
        _ptr(topk_idx, "topk_idx", torch.int64) if topk_idx.numel() else None,
        ctypes.byref(layout.struct), layout.workspace.data_ptr(), layout.workspace.numel(),
        _ptr(x, "x", xt), H, recv_dtype, _ptr(recv_x, "recv_x", rt),
        _ptr(recv_scales, "recv_scales", st), _stream(stream)))
    return layout


def ep_combine(expert_out: torch.Tensor, topk_weights: torch.Tensor, layout: EpLayout,
               out: torch.Tensor, stream=None) -> None:
    """expert_out bf16 [R, H], topk_weights fp32 [T, k] -> out bf16 [T, H]."""
    H = expert_out.shape[-1]
    if (tuple(expert_out.shape) != (layout.num_recv_rows, H)
            or tuple(topk_weights.shape) != (layout.num_tokens, layout.num_topk)
            or tuple(out.shape) != (layout.num_tokens, H)):
        raise ValueError("combine buffers do not match the layout")
    _check("ep_combine", lib().ep_combine(
        _ptr(expert_out, "expert_out", torch.bfloat16), _ptr(topk_weights, "topk_weights", torch.float32),
        ctypes.byref(layout.struct), H, _ptr(out, "out", torch.bfloat16), _stream(stream)))


def ep_combine_f16(expert_out: torch.Tensor, topk_weights: torch.Tensor, layout: EpLayout,
                   out: torch.Tensor, stream=None) -> None:
    """expert_out fp16 [R, H], topk_weights fp32 [T, k] -> out fp16 [T, H]."""
    H = expert_out.shape[-1]
    if (tuple(expert_out.shape) != (layout.num_recv_rows, H)
            or tuple(topk_weights.shape) != (layout.num_tokens, layout.num_topk)
            or tuple(out.shape) != (layout.num_tokens, H)):
        raise ValueError("combine buffers do not match the layout")
    _check("ep_combine_f16", lib().ep_combine_f16(
        _ptr(expert_out, "expert_out", torch.float16), _ptr(topk_weights, "topk_weights", torch.float32),
        ctypes.byref(layout.struct), H, _ptr(out, "out", torch.float16), _stream(stream)))


def ep_combine_fp8(expert_q: torch.Tensor, expert_scales: torch.Tensor, topk_weights: torch.Tensor,
                   layout: EpLayout, out: torch.Tensor, stream=None) -> None:
    """expert_q uint8 [R, H] E4M3 codes, expert_scales fp32 [R, H/128],
    topk_weights fp32 [T, k] -> out bf16 [T, H]."""
    H = expert_q.shape[-1]
    if (tuple(expert_q.shape) != (layout.num_recv_rows, H)
            or tuple(expert_scales.shape) != (layout.num_recv_rows, H // 128)
            or tuple(topk_weights.shape) != (layout.num_tokens, layout.num_topk)
            or tuple(out.shape) != (layout.num_tokens, H)):
        raise ValueError("combine buffers do not match the layout")
    _check("ep_combine_fp8", lib().ep_combine_fp8(
        _ptr(expert_q, "expert_q", torch.uint8), _ptr(expert_scales, "expert_scales", torch.float32),
        _ptr(topk_weights, "topk_weights", torch.float32), ctypes.byref(layout.struct), H,
        _ptr(out, "out", torch.bfloat16), _stream(stream)))


def ep_combine_mxfp8(expert_q: torch.Tensor, expert_scales: torch.Tensor, topk_weights: torch.Tensor,
                     layout: EpLayout, out: torch.Tensor, stream=None) -> None:
    """expert_q uint8 [R, H] E4M3 codes, expert_scales uint8 [R, H/32] E8M0 bytes,
    topk_weights fp32 [T, k] -> out bf16 [T, H]."""
    H = expert_q.shape[-1]
    if (tuple(expert_q.shape) != (layout.num_recv_rows, H)
            or tuple(expert_scales.shape) != (layout.num_recv_rows, H // 32)
            or tuple(topk_weights.shape) != (layout.num_tokens, layout.num_topk)
            or tuple(out.shape) != (layout.num_tokens, H)):
        raise ValueError("combine buffers do not match the layout")
    _check("ep_combine_mxfp8", lib().ep_combine_mxfp8(
        _ptr(expert_q, "expert_q", torch.uint8), _ptr(expert_scales, "expert_scales", torch.uint8),
        _ptr(topk_weights, "topk_weights", torch.float32), ctypes.byref(layout.struct), H,
        _ptr(out, "out", torch.bfloat16), _stream(stream)))


def ep_get_group_layout(topk_idx: torch.Tensor, topk_weights: torch.Tensor | None,
                        layout: EpGroupLayout, recv_topk_idx: torch.Tensor | None = None,
                        recv_topk_weights: torch.Tensor | None = None, stream=None,
                        is_token_in_group: torch.Tensor | None = None) -> EpGroupLayout:
    """topk_idx int64 [T, k] (and topk_weights fp32 [T, k] when
    recv_topk_weights is wanted) -> the group layout's arrays, plus optional
    recv_topk_idx int64 [T*kg, k] / recv_topk_weights fp32 [T*kg, k] and
    is_token_in_group uint8 (or bool) [T, G]."""
    T, k = layout.num_tokens, layout.source_topk
    if tuple(topk_idx.shape) != (T, k):
        raise ValueError("topk_idx shape %s does not match the layout" % (tuple(topk_idx.shape),))
    rows = (layout.num_recv_rows, k)
    for name, t in (("topk_weights", topk_weights),):
        if t is not None and tuple(t.shape) != (T, k):
            raise ValueError("%s shape does not match the layout" % name)
    for name, t in (("recv_topk_idx", recv_topk_idx), ("recv_topk_weights", recv_topk_weights)):
        if t is not None and tuple(t.shape) != rows:
            raise ValueError("%s must have shape %s" % (name, rows))
    member = None
    if is_token_in_group is not None:
        if tuple(is_token_in_group.shape) != (T, layout.num_experts):
            raise ValueError("is_token_in_group must have shape %s" % ((T, layout.num_experts),))
        member = is_token_in_group.view(torch.uint8) if is_token_in_group.dtype == torch.bool else is_token_in_group
    _check("ep_get_group_layout", lib().ep_get_group_layout(
        _ptr(topk_idx, "topk_idx", torch.int64) if topk_idx.numel() else None,
        _ptr(topk_weights, "topk_weights", torch.float32) if topk_weights is not None and topk_weights.numel() else None,
        k, layout.source_experts, ctypes.byref(layout.struct),
        _ptr(recv_topk_idx, "recv_topk_idx", torch.int64) if recv_topk_idx is not None and recv_topk_idx.numel() else None,
        _ptr(recv_topk_weights, "recv_topk_weights", torch.float32) if recv_topk_weights is not None and recv_topk_weights.numel() else None,
        _ptr(member, "is_token_in_group", torch.uint8) if member is not None and member.numel() else None,
        layout.workspace.data_ptr(), layout.workspace.numel(), _stream(stream)))
    return layout


def ep_combine_groups(z: torch.Tensor, layout: EpGroupLayout, out: torch.Tensor,
                      stream=None) -> None:
    """z bf16 [T*kg, H] (one already-weighted row per (token, group)) -> out
    bf16 [T, H], the unit-weight sum of each token's group rows."""
    H = z.shape[-1]
    if tuple(z.shape) != (layout.num_recv_rows, H) or tuple(out.shape) != (layout.num_tokens, H):
        raise ValueError("group combine buffers do not match the layout")
    _check("ep_combine_groups", lib().ep_combine_groups(
        _ptr(z, "z", torch.bfloat16), ctypes.byref(layout.struct), H,
        _ptr(out, "out", torch.bfloat16), _stream(stream)))


def ep_dequant_fp8(q: torch.Tensor, scales: torch.Tensor, y: torch.Tensor, stream=None) -> None:
    rows, H = q.shape
    if tuple(y.shape) != (rows, H) or tuple(scales.shape) != (rows, H // 128):
        raise ValueError("dequant buffers disagree")
    _check("ep_dequant_fp8", lib().ep_dequant_fp8(
        _ptr(q, "q", torch.uint8), _ptr(scales, "scales", torch.float32), rows, H,
        _ptr(y, "y", torch.bfloat16), _stream(stream)))


def ep_dequant_mxfp8(q: torch.Tensor, scales: torch.Tensor, y: torch.Tensor, stream=None) -> None:
    rows, H = q.shape
    if tuple(y.shape) != (rows, H) or tuple(scales.shape) != (rows, H // 32):
        raise ValueError("dequant buffers disagree")
    _check("ep_dequant_mxfp8", lib().ep_dequant_mxfp8(
        _ptr(q, "q", torch.uint8), _ptr(scales, "scales", torch.uint8), rows, H,
        _ptr(y, "y", torch.bfloat16), _stream(stream)))


def ep_scales_to_mn_major(scales: torch.Tensor, hidden: int, recv_dtype: int, scales_mn: torch.Tensor,
                          stream=None) -> None:
    """Row-major scales of an FP8 dispatch (fp32 [R, H/128] or MXFP8 uint8
    [R, H/32]) -> their MN-major layout ([H/128, R] or [H/32, R])."""
    recv_dtype &= ~EP_SCALES_MN_MAJOR
    if recv_dtype not in _FP8_DTYPES:
        raise ValueError("recv_dtype %d has no scales" % recv_dtype)
    per_row = hidden // 32 if recv_dtype == EP_MXFP8_E4M3 else hidden // 128
    rows = scales.shape[0]
    if tuple(scales.shape) != (rows, per_row) or tuple(scales_mn.shape) != (per_row, rows):
        raise ValueError("scale buffers disagree: %s -> %s" % (tuple(scales.shape), tuple(scales_mn.shape)))
    st = torch.uint8 if recv_dtype == EP_MXFP8_E4M3 else torch.float32
    _check("ep_scales_to_mn_major", lib().ep_scales_to_mn_major(
        _ptr(scales, "scales", st), rows, hidden, recv_dtype, _ptr(scales_mn, "scales_mn", st),
        _stream(stream)))


def ep_cast_e4m3_bits(first: int, n: int, method: int, out: torch.Tensor, stream=None) -> None:
    if out.numel() < n:
        raise ValueError("out too small")
    _check("ep_cast_e4m3_bits", lib().ep_cast_e4m3_bits(
        first & 0xFFFFFFFF, n, method, _ptr(out, "out", torch.uint8), _stream(stream)))


def ep_copy(src: torch.Tensor, dst: torch.Tensor, stream=None) -> None:
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("dst too small")
    _check("ep_copy", lib().ep_copy(_ptr(src, "src"), _ptr(dst, "dst"), nbytes, _stream(stream)))


def ep_version() -> str:
    return lib().ep_version().decode()
