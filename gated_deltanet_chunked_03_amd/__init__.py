"""Gated DeltaNet chunked prefill for AMD MI355X (gfx950): the forward with
gate-driven intra-card context parallelism, its backward, a recurrent decode
step and a segment-length calibration.

Everything runs in hand-written HIP kernels behind a C ABI (include/gdn.h,
built into _build/libgdn.so); this package is the thin Python binding over it
plus a seeded synthetic-input generator.
"""
from .binding import (GDNError, bwd, calibrate_lambda, chunk_gated_delta_rule, chunk_prep,  # noqa: F401
                      decode, fwd, load_library, plan, profile_enable, profile_read, LIB_PATH)
