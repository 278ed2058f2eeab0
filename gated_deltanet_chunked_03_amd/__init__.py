"""Gated DeltaNet chunked-prefill forward for AMD MI355X (gfx950).

The forward runs in hand-written HIP kernels behind a C ABI (include/gdn.h,
built into _build/libgdn.so); this package is the thin Python binding over it
plus a seeded synthetic-input generator.
"""
from .binding import (GDNError, bwd, chunk_gated_delta_rule, chunk_prep, decode, fwd, load_library,  # noqa: F401
                      plan, profile_enable, profile_read, LIB_PATH)
