"""LDS-poisoning build against the normal build.

``_build/libgdn_poison.so`` is compiled from the same sources with
GDN_LDS_POISON: every kernel first fills its shared memory with 0xFFFFFFFF
words (NaN as fp32, fp16 and bf16; -1 as an int). If any kernel read LDS that
no thread of its workgroup had written, its results would change. Each case
below runs one call through both builds on the same inputs: the forward
kernels are deterministic, so their outputs must agree bit for bit; the
backward's chunk kernel sums some row terms with LDS atomics in wave order,
so its outputs are compared to 1e-5 relative. Every output is also checked
to be finite. The cases cover each kernel: T diag(beta) preparation (both
image kinds), the CP preprocessing in both layouts and for fp32 inputs, the
boundary-state chains (single and grouped), the fused forward in every column split, the debug
copies, the backward's kernels and the decode.
"""
from __future__ import annotations

import contextlib
import os

import numpy as np
import pytest

from gated_deltanet_chunked_03_amd.synth import make_inputs
from gpu_util import to_device

pytestmark = pytest.mark.gpu

POISON_LIB = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                          "gated_deltanet_chunked_03_amd", "_build", "libgdn_poison.so")


@contextlib.contextmanager
def _library(path):
    from gated_deltanet_chunked_03_amd import binding
    binding.load_library()
    saved = binding._lib
    binding._lib = binding.load_library(path) if path else saved
    try:
        yield
    finally:
        binding._lib = saved


def _both(fn):
    """fn() under the normal build, then under the poisoned build (numpy results)."""
    import torch
    out = []
    for path in (None, POISON_LIB):
        with _library(path):
            res = fn()
            torch.cuda.synchronize()
        out.append(res)
    return out


def _np(x):
    return None if x is None else x.float().cpu().numpy()


def _same(a, b, what, exact=True):
    for key in a:
        x, y = a[key], b[key]
        if x is None:
            assert y is None, (what, key)
            continue
        assert np.isfinite(x).all() and np.isfinite(y).all(), f"{what}: {key} not finite"
        if exact:
            assert np.array_equal(x, y), f"{what}: {key} differs between the builds"
        else:
            scale = max(float(np.abs(x).max()), 1e-30)
            assert float(np.abs(x - y).max()) <= 1e-5 * scale, f"{what}: {key} differs between the builds"


def _boundary_slots(inp, L):
    """Segment slots that hold a boundary state (every segment but each sequence's first)."""
    lens = np.diff(np.asarray(inp.cu_seqlens)) if inp.cu_seqlens is not None else [inp.T] * inp.B
    slots, base = [], 0
    for n in lens:
        N = -(-int(n) // 64)
        P = 1 if N == 0 else -(-N // L)
        slots += list(range(base + 1, base + P))
        base += P
    return slots


def _fwd_case(inp, **kw):
    import gated_deltanet_chunked_03_amd as gdn

    def run():
        d = to_device(inp)
        o, S, info = gdn.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], scale=inp.scale,
                             initial_state=d["initial_state"], cu_seqlens=inp.cu_seqlens, debug=True, **kw)
        res = {"o": _np(o), "S": _np(S)}
        if info["plan"]["cp_on"]:
            res["seg"] = _np(info["seg_state"])[_boundary_slots(inp, info["plan"]["L"])]
            res["path"] = info["path"].cpu().numpy()
        return res
    return run


def test_poison_lib_built():
    assert os.path.exists(POISON_LIB), "build() writes the LDS-poisoning library beside libgdn.so"


@pytest.mark.parametrize("case", [
    dict(io="bf16", T=333, h=(2, 4), kw=dict(cp_mode="off")),
    dict(io="f32", T=512, h=(1, 1), kw=dict(cp_mode="off")),
    dict(io="bf16", T=64 * 40 + 5, h=(2, 8), kw=dict(cp_mode="auto", n_cu=32, lam=0.6, cp_layout=1)),
    dict(io="bf16", T=64 * 40 + 5, h=(2, 8), kw=dict(cp_mode="exact", n_cu=32, lam=0.6, cp_layout=2)),
    dict(io="bf16", T=64 * 40 + 5, h=(2, 8), kw=dict(cp_mode="warmup", n_cu=32, lam=0.6, cp_layout=2)),
    dict(io="f32", T=64 * 40 + 5, h=(2, 8), kw=dict(cp_mode="auto", n_cu=32, lam=0.6)),
    dict(io="bf16", T=64 * 9 + 17, h=(2, 4), kw=dict(cp_mode="off", dv_split=2)),
    dict(io="bf16", T=64 * 9 + 17, h=(2, 4), kw=dict(cp_mode="off", dv_split=4)),
], ids=["bf16-off", "f32-off", "auto-layout1", "exact-layout2", "warmup-layout2", "f32-auto", "dv2", "dv4"])
def test_forward_same_under_poison(case):
    inp = make_inputs(1, case["T"], *case["h"], seed=90, gate="mixed", init_std=0.05, io_dtype=case["io"])
    a, b = _both(_fwd_case(inp, **case["kw"]))
    _same(a, b, f"fwd {case['io']} {case['kw']}")


def test_grouped_combine_same_under_poison():
    """Long boundary chains, so that the planner groups the combine (composed
    group maps, then the replay)."""
    from gated_deltanet_chunked_03_amd import plan
    cu = [0, 64 * 129 + 37, 64 * 129 + 37 + 64 * 70 + 5]
    inp = make_inputs(1, cu[-1], 2, 4, seed=95, gate="mixed", cu_seqlens=cu, init_std=0.05)
    for mode in ("exact", "auto"):
        assert plan(1, cu[-1], 2, 4, cu_seqlens=cu, cp_mode=mode, n_cu=256)["combine_group"] > 0
        a, b = _both(_fwd_case(inp, cp_mode=mode, n_cu=256))
        _same(a, b, f"grouped combine {mode}")


def test_varlen_same_under_poison():
    cu = [0, 700, 700, 701, 64 * 20 + 3, 64 * 20 + 3 + 130]
    inp = make_inputs(1, cu[-1], 1, 4, seed=91, gate="mixed", cu_seqlens=cu, init_std=0.1)
    for layout in (1, 2):
        a, b = _both(_fwd_case(inp, cp_mode="auto", n_cu=64, lam=0.5, warmup_chunks=2, cp_layout=layout))
        _same(a, b, f"varlen layout {layout}")


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_chunk_prep_same_under_poison(io):
    import gated_deltanet_chunked_03_amd as gdn
    inp = make_inputs(1, 64 * 5 + 9, 1, 3, seed=92, gate="mixed", io_dtype=io)

    def run():
        d = to_device(inp)
        gam, W, U = gdn.chunk_prep(d["k"], d["v"], d["g"], d["beta"])
        return {"gamma": _np(gam), "W": _np(W), "U": _np(U)}
    a, b = _both(run)
    _same(a, b, f"chunk_prep {io}")


@pytest.mark.parametrize("mode", ["off", "auto"])
def test_backward_same_under_poison(mode):
    import torch
    import gated_deltanet_chunked_03_amd as gdn
    inp = make_inputs(1, 64 * 21 + 23, 2, 4, seed=93, gate="mixed", init_std=0.1)
    r = np.random.default_rng(193)
    d_out = r.standard_normal(inp.v.shape).astype(np.float32)
    d_fin = (0.1 * r.standard_normal((1, inp.h_v, 128, 128))).astype(np.float32)

    def run():
        d = to_device(inp)
        res = gdn.bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], torch.from_numpy(d_out).to("cuda", torch.bfloat16),
                      scale=inp.scale, initial_state=d["initial_state"],
                      d_final_state=torch.from_numpy(d_fin).cuda(), cp_mode=mode, n_cu=16, lam=0.5,
                      warmup_chunks=2)
        return {k: _np(x) for k, x in res.items()}
    a, b = _both(run)
    _same(a, b, f"bwd {mode}", exact=False)


def test_decode_same_under_poison():
    import gated_deltanet_chunked_03_amd as gdn
    inp = make_inputs(3, 5, 2, 4, seed=94, gate="mixed", init_std=0.1)

    def run():
        d = to_device(inp)
        o, S = gdn.decode(d["q"], d["k"], d["v"], d["g"], d["beta"], d["initial_state"], scale=inp.scale)
        return {"o": _np(o), "S": _np(S)}
    a, b = _both(run)
    _same(a, b, "decode")
