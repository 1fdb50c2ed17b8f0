"""Block-sparse long-context decode attention for AMD MI355X (gfx950).

The compute lives in libkvs.so (hand-written HIP kernels behind a C ABI, include/kvs.h); this
package is its ctypes binding plus a small torch-facing helper layer (``ops``) that allocates
outputs and workspaces as torch tensors.
"""
from .binding import *  # noqa: F401,F403
from .binding import Config, KvsError, LIB_PATH, EXPORTS  # noqa: F401
from . import ops  # noqa: F401
