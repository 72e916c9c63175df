"""MI355X-native MoE token dispatch / combine (layout -> dispatch -> combine).

The compute path is a C-ABI shared library of hand-written HIP kernels for
gfx950 (``libep.so``, declared in ``include/ep.h``); ``binding`` marshals torch
tensors into it.  Importing this package loads nothing: the library is opened
on first use and a missing library is an error, never a fallback.
"""
__version__ = "0.1.0"
