"""fp64 CPU oracle of the Gated DeltaNet chunked-prefill forward (test infrastructure).

Only the tests, the smoke check and the benchmark's CPU-baseline leg import this
package. The library in ``gated_deltanet_chunked_03_amd`` never imports it and the
two share no code.

Modules:
  sequential   -- token-by-token recurrence: C (threaded, timed) and numpy forms
  exact        -- exact rational brute force of the matrix-product form (tiny inputs)
  chunk_model  -- fp64 chunked (WY) form with exact and warm-up context parallelism
  backward     -- fp64 gradients of the recurrence: C (threaded) and numpy forms
"""
from .sequential import build, gdn_sequential, gdn_sequential_np, lib_path  # noqa: F401
from .exact import gdn_exact_fraction  # noqa: F401
from . import chunk_model  # noqa: F401
from .backward import gdn_sequential_bwd, gdn_sequential_bwd_np  # noqa: F401
