"""Skinny draft-head vocabulary projection for MI355X (gfx950).

The compute lives in liblmhead.so (HIP kernels behind the C ABI of
include/lmhead.h); this package is its Python binding.
"""
from .lmhead import *  # noqa: F401,F403
from .lmhead import __all__  # noqa: F401
