"""MI355X-native routed MoE expert-layer forward with an HBM expert cache.

The compute path is libmoe.so (HIP kernels for gfx950 behind the C ABI in
include/moe.h); :mod:`.binding` marshals arguments to it and :mod:`.engine`
wraps a context for Python callers.  Importing this package loads the
library and raises ImportError when it has not been built.
"""
from .binding import MoEError, lib  # noqa: F401
from .engine import MoEEngine  # noqa: F401
