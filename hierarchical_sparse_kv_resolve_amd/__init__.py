"""MI355X (gfx950) sparse KV row resolver: HIP kernels behind a C ABI (libkvr.so)
with a thin ctypes binding.  See include/kvr.h for the calls."""
from . import kvr  # noqa: F401
from .kvr import Context, KvrError  # noqa: F401
