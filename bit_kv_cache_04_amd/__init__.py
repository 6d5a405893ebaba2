"""Low-bit KV-cache append and decode attention for MI355X (gfx950).

libkvq.so (built from csrc/ by `_build.build()`) holds every kernel and the C
ABI declared in include/kvq.h; `kvq` binds it with ctypes under the same
names, and `cache.PackedKVCache` keeps a cache's buffers in torch device
memory.  Importing the package does not load the library; the first call does,
and fails loudly if it has not been built.
"""

from . import kvq  # noqa: F401
