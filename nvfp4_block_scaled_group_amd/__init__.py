"""Grouped, row-scaled (per-token) NVFP4 amax + cast for packed MoE
activations on MI355X (gfx950).

The work is done by hand-written HIP kernels behind a C-ABI library
(``libnvfp4g.so``, declared in ``include/nvfp4_group.h``); ``binding`` is a thin
ctypes layer with the same entry-point names.  Importing this package loads
nothing: the library is loaded on first use, and a missing library is an error.
"""
__all__ = ["binding", "synth"]
