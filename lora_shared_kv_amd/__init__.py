"""Shared-prefix multi-LoRA attention for MI355X (gfx950).

The compute path is the native library libskv.so (C ABI in include/skv.h,
HIP kernels for gfx950); this package is its Python binding.
"""
from .skv import *  # noqa: F401,F403
from .skv import (SKV_BASE_LR_SHARED, SKV_BASE_SHARED, SKV_SHARED, Ctx, SkvError,  # noqa: F401
                  load_library, library_path)
