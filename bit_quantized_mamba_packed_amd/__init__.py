"""DF-SSM inference hot path for AMD MI355X (gfx950): HIP kernels behind a C ABI (libdfssm.so).

`_lib` is the ctypes binding of include/dfssm.h; `device` marshals torch device tensors into it.
"""
from . import _lib  # noqa: F401

__all__ = ["_lib"]
