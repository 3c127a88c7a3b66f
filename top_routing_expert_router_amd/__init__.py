"""MI355X (gfx950) token-choice MoE FFN layer forward.

The layer runs in hand-written HIP kernels behind the C ABI of include/moe.h
(libmoe_hip.so); `binding` is the thin ctypes layer over it.  Importing this
package loads nothing; the first binding call loads the library and fails
loudly if it has not been built.
"""
from . import binding  # noqa: F401
from .binding import MoEConfig, MoEError  # noqa: F401
