"""MI355X-native MoE token dispatch / combine (layout -> dispatch -> combine).

The compute path is a C-ABI shared library of hand-written HIP kernels for
gfx950 (``libep.so``, declared in ``include/ep.h``); ``binding`` marshals torch
tensors into it under the same names.  Importing this package loads nothing:
the library is opened on first use and a missing library is an error, never a
fallback.
"""
from .binding import (EP_BF16, EP_F16, EP_FLAG_BAD_EXPERT, EP_FLAG_OVERFLOW, EP_FP8_E4M3,
                      EP_FP8_E4M3_POW2, EP_MXFP8_E4M3, EP_SCALES_MN_MAJOR, EpError,
                      EpGroupLayout, EpLayout,
                      ep_cast_e4m3_bits, ep_combine, ep_combine_f16, ep_combine_fp8, ep_combine_mxfp8,
                      ep_combine_groups, ep_copy, ep_dequant_fp8, ep_dequant_mxfp8, ep_dispatch,
                      ep_get_group_layout, ep_get_layout, ep_layout_dispatch,
                      ep_layout_workspace_bytes, ep_num_recv_rows, ep_scales_to_mn_major,
                      ep_version)

__version__ = "0.1.0"
