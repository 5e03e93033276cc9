"""Routed MoE FFN layer with a resident-expert cache, native to MI355X (gfx950).

The compute path is the HIP library ``libftmoe.so`` (C ABI in
``include/ft_moe.h``); ``ops`` binds its entry points one to one and
``layer`` holds device buffers and the per-layer call sequence.  Importing
this package does not load the library; the first call does, and raises if
it has not been built.
"""
from . import _lib  # noqa: F401

__all__ = ["ops", "layer", "build"]
