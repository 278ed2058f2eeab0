"""Helpers shared by the GPU parity tests: device copies of seeded inputs, the
oracle run on the same values, and the error metrics the tolerance is stated in.

Tolerance (stated for bf16 inputs; also applied to fp32 inputs):
    max |o - o_ref| <= 1e-2 * max |o_ref|
    sum |o - o_ref| / sum |o_ref| <= 2e-3      (mean relative error, as relative L1)
o_ref is the fp64 sequential oracle on exactly the values the GPU sees.

States (final states and segment boundary states) are checked at 1e-3
relative, the bound the target states for the warm-up path's extra state
error: the forward's chain runs on fp16 matrix-core operands (every derived
operand rounded once to an 11-bit significand), which leaves states about
5e-4 off (measured in a CPU model of that rounding), exact and warm-up
boundaries alike.
"""
from __future__ import annotations

import numpy as np

from oracle import gdn_sequential

MAX_TOL = 1e-2
MEAN_TOL = 2e-3
STATE_MAX_TOL = 2e-3    # max |S - S_ref| / max |S_ref|
STATE_MEAN_TOL = 1e-3   # sum |S - S_ref| / sum |S_ref|
BOUNDARY_TOL = 1e-3     # ||S0 - S0_ref||_F / ||S0_ref||_F per boundary, exact or warm-up


def to_device(inp, device="cuda"):
    import torch
    dt = torch.bfloat16 if inp.io_dtype == "bf16" else torch.float32
    t = lambda a, d=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to(device=device, dtype=d)  # noqa
    dev = dict(q=t(inp.q, dt), k=t(inp.k, dt), v=t(inp.v, dt), g=t(inp.g), beta=t(inp.beta))
    dev["initial_state"] = None if inp.initial_state is None else t(inp.initial_state)
    return dev


def oracle_run(inp, snap_stride=0, n_snap=0, n_threads=None):
    q, k, v, g, b = inp.flat()
    return gdn_sequential(q, k, v, g, b, inp.scale, inp.initial_state, inp.flat_cu(),
                          snap_stride=snap_stride, n_snap=n_snap, n_threads=n_threads)


def errors(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    d = np.abs(x - ref)
    return float(d.max() / max(np.abs(ref).max(), 1e-30)), float(d.sum() / max(np.abs(ref).sum(), 1e-30))


def assert_within_tolerance(x, ref, what="o", max_tol=MAX_TOL, mean_tol=MEAN_TOL):
    mx, mean = errors(x, ref)
    assert np.all(np.isfinite(x)), f"{what}: non-finite values"
    assert mx <= max_tol and mean <= mean_tol, \
        f"{what}: max-rel {mx:.3e} (tol {max_tol:g}), mean-rel {mean:.3e} (tol {mean_tol:g})"
    return mx, mean
