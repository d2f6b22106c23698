"""MI355X-native small-batch decode step with tile-flag overlapped stages.

The compute path is libld.so (hand-written HIP for gfx950); `ld` is its thin
ctypes binding.  Importing fails when the library has not been built.
"""
from . import ld  # noqa: F401
from .ld import Model  # noqa: F401
