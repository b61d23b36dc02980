"""MI355X-native (gfx950) expert-parallel MoE dispatch / combine core.

The work is done by the HIP kernels in ``libep.so`` behind the C ABI of
``include/ep.h``; ``combine_get_layout_amd.ep`` is the ctypes binding with the
same entry-point names. Build with ``python -m combine_get_layout_amd.build``.
"""
from . import ep  # noqa: F401  (loads libep.so lazily, on first call)

__all__ = ["ep"]
