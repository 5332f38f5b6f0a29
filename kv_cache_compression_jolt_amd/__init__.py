"""JoLT per-layer-group KV-cache compressor for MI355X (gfx950).

The compute path is libjolt.so (HIP kernels behind a C ABI, see
include/libjolt.h); this package holds its sources (csrc/), the build script and
the ctypes binding.
"""
from .binding import (  # noqa: F401
    Jolt,
    JoltError,
    jolt_alloc,
    jolt_config,
    jolt_item,
    make_config,
    make_item,
)
