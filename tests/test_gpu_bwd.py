"""Backward pass (gdn_bwd) against the fp64 backward oracle.

The oracle is the gradient of the sequential recurrence (oracle/backward.py,
pinned by finite differences); both sides see the same bf16-rounded inputs and
the same loss gradients (fp32 inputs: see the fp32 cases below). Tolerances: the bf16 outputs dq, dk, dv take the
forward's bound (max |x - x_ref| <= 1e-2 max |x_ref|, relative L1 <= 2e-3: bf16
rounding of the result alone costs about 1.4e-3); the fp32 outputs dg, dbeta
and the initial-state gradient carry only fp32 arithmetic and the forward
re-run's state error (about 1e-5 relative), so they are held to max 1e-3 and
relative L1 1e-4. With AutoCP warm-up boundaries the re-run's states differ
from the exact ones by at most the noise floor (1e-4 relative), inside both.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest

from gated_deltanet_chunked_03_amd.synth import make_inputs, round_bf16
from gpu_util import assert_within_tolerance, to_device
from oracle import gdn_sequential_bwd

pytestmark = pytest.mark.gpu

F32_MAX, F32_MEAN = 1e-3, 1e-4


def _grads(seed, shape_o, n_seqs, h_v, with_final=True, io="bf16"):
    r = np.random.default_rng(seed)
    d_out = r.standard_normal(shape_o).astype(np.float32)
    if io == "bf16":
        d_out = round_bf16(d_out).astype(np.float32)
    d_fin = (0.1 * r.standard_normal((n_seqs, h_v, 128, 128))).astype(np.float32) if with_final else None
    return d_out, d_fin


def _run(inp, d_out, d_fin, **kw):
    import torch
    import gated_deltanet_chunked_03_amd as gdn
    d = to_device(inp)
    dd = torch.from_numpy(d_out).to("cuda", torch.bfloat16 if inp.io_dtype == "bf16" else torch.float32)
    df = None if d_fin is None else torch.from_numpy(d_fin).cuda()
    cu = None if inp.cu_seqlens is None else [int(x) for x in inp.cu_seqlens]
    res = gdn.bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], dd, scale=inp.scale,
                  initial_state=d["initial_state"], d_final_state=df, cu_seqlens=cu, **kw)
    torch.cuda.synchronize()
    for key in ("dq", "dk", "dv"):
        assert res[key].dtype == d["q"].dtype, (key, res[key].dtype)
    return {k: (None if x is None else x.float().cpu().numpy()) for k, x in res.items()}


def _check(inp, d_out, d_fin, got, what, f32_tol=(F32_MAX, F32_MEAN), io_tol=()):
    q, k, v, g, b = inp.flat()
    BT = inp.B * inp.T
    ref = gdn_sequential_bwd(q, k, v, g, b, inp.scale, d_out.reshape(BT, inp.h_v, -1), inp.initial_state,
                             d_fin, inp.flat_cu())
    shape = lambda x, ref_x: x.reshape(ref_x.shape)  # noqa: E731
    errs = {}
    for key in ("dq", "dk", "dv"):
        errs[key] = assert_within_tolerance(shape(got[key], ref[key]), ref[key], f"{what}: {key}", *io_tol)
    for key in ("dg", "dbeta"):
        errs[key] = assert_within_tolerance(shape(got[key], ref[key]), ref[key], f"{what}: {key}", *f32_tol)
    if got["d_initial"] is not None:
        errs["d_initial"] = assert_within_tolerance(got["d_initial"], ref["d_initial"], f"{what}: d_initial",
                                                    *f32_tol)
    print(f"[{what}] " + " ".join(f"{k} {m:.2e}/{a:.2e}" for k, (m, a) in errs.items()), flush=True)


@pytest.mark.parametrize("mode", ["off", "exact"])
def test_bwd_single_sequence(mode):
    inp = make_inputs(name="bwd1", B=1, T=64 * 5 + 23, h_qk=2, h_v=4, seed=31, gate="mixed", init_std=0.1)
    print(f"\n[bwd/single/{mode}] T={inp.T}", flush=True)
    d_out, d_fin = _grads(131, inp.v.shape, 1, inp.h_v)
    got = _run(inp, d_out, d_fin, cp_mode=mode, n_cu=8)
    _check(inp, d_out, d_fin, got, f"single/{mode}")


def test_bwd_batch_no_state_gradients():
    inp = make_inputs(name="bwdB", B=3, T=150, h_qk=1, h_v=2, seed=32, gate="plain")
    print("\n[bwd/batch] B=3 T=150, no initial state, no final-state gradient", flush=True)
    d_out, _ = _grads(132, inp.v.shape, 3, inp.h_v, with_final=False)
    got = _run(inp, d_out, None)
    _check(inp, d_out, None, got, "batch")


def test_bwd_varlen_auto_cp():
    cu = [0, 64 * 9 + 5, 64 * 9 + 5, 64 * 9 + 5 + 64 * 20 + 40]   # includes an empty sequence
    inp = make_inputs(name="bwdV", B=1, T=cu[-1], h_qk=2, h_v=4, seed=33, gate="mixed", init_std=0.1,
                      cu_seqlens=cu)
    print(f"\n[bwd/varlen] cu={cu}, AutoCP on 32 CUs", flush=True)
    d_out, d_fin = _grads(133, inp.v.shape, 3, inp.h_v)
    got = _run(inp, d_out, d_fin, cp_mode="auto", n_cu=32, lam=0.5, warmup_chunks=2)
    _check(inp, d_out, d_fin, got, "varlen")
    # the empty sequence passes its state gradient through
    np.testing.assert_array_equal(got["d_initial"][1], d_fin[1])


def test_bwd_items_past_one_round():
    """More (chunk, head) items than the chunk-gradient kernel has workgroups
    (one per CU) and not a multiple of them: 71 chunks x 4 heads = 284 items,
    so some workgroups take a second item (and fetch it during the first)."""
    inp = make_inputs(name="bwdR", B=1, T=64 * 70 + 9, h_qk=1, h_v=4, seed=36, gate="mixed", init_std=0.1)
    print(f"\n[bwd/items] T={inp.T}", flush=True)
    d_out, d_fin = _grads(136, inp.v.shape, 1, inp.h_v)
    got = _run(inp, d_out, d_fin, cp_mode="auto", n_cu=64, lam=0.5)
    _check(inp, d_out, d_fin, got, "items past one round")


# fp32 inputs are rounded once to bf16 inside the backward, which then runs as
# for bf16 inputs and writes every gradient in fp32. Two checks: against the
# oracle's gradient at the rounded inputs, every output (dq, dk, dv now fp32
# too) is held to the fp32 bound above -- the kernels add nothing beyond that;
# against the gradient at the fp32 inputs themselves, each output carries the
# input rounding: RNE to bf16 costs about 1.4e-3 relative L1 per rounded tensor
# (what bf16 rounding of the outputs alone costs above), and a gradient is
# multilinear in up to four rounded tensors (q, k, v, dO) whose independent
# errors add in quadrature (about 2.8e-3), so relative L1 5e-3 and the
# forward's max bound.
BF16_IN = (1e-2, 5e-3)


def _rounded(inp):
    rb = lambda a: round_bf16(a).astype(np.float32)  # noqa: E731
    return dataclasses.replace(inp, q=rb(inp.q), k=rb(inp.k), v=rb(inp.v))


def _check_fp32_inputs(inp, d_out, d_fin, got, what):
    _check(_rounded(inp), round_bf16(d_out).astype(np.float32), d_fin, got, f"{what} (rounded inputs)",
           (F32_MAX, F32_MEAN), (F32_MAX, F32_MEAN))
    _check(inp, d_out, d_fin, got, what, BF16_IN, BF16_IN)


@pytest.mark.parametrize("mode", ["off", "exact", "auto"])
def test_bwd_fp32_inputs(mode):
    inp = make_inputs(name="bwd32", B=1, T=64 * 6 + 41, h_qk=2, h_v=4, seed=34, gate="mixed", init_std=0.1,
                      io_dtype="f32")
    print(f"\n[bwd/fp32/{mode}] T={inp.T}", flush=True)
    d_out, d_fin = _grads(134, inp.v.shape, 1, inp.h_v, io="f32")
    got = _run(inp, d_out, d_fin, cp_mode=mode, n_cu=8, lam=0.5, warmup_chunks=2)
    _check_fp32_inputs(inp, d_out, d_fin, got, f"fp32/{mode}")


def test_bwd_fp32_varlen():
    cu = [0, 64 * 3 + 7, 64 * 3 + 7, 64 * 3 + 8, 64 * 11 + 30]
    inp = make_inputs(name="bwd32V", B=1, T=cu[-1], h_qk=1, h_v=2, seed=35, gate="mixed", init_std=0.1,
                      cu_seqlens=cu, io_dtype="f32")
    print(f"\n[bwd/fp32/varlen] cu={cu}", flush=True)
    d_out, d_fin = _grads(135, inp.v.shape, len(cu) - 1, inp.h_v, io="f32")
    got = _run(inp, d_out, d_fin, cp_mode="auto", n_cu=8, lam=0.5, warmup_chunks=2)
    _check_fp32_inputs(inp, d_out, d_fin, got, "fp32/varlen")


def test_bwd_varlen_many_items():
    """Variable-length sequences with more (chunk, head) items than the
    persistent prep (two workgroups per CU) and chunk-gradient kernel (one per
    CU) have workgroups: three sequences, 533 chunks x 8 value heads = 4264
    items, so each workgroup takes several items, of different sequences
    (located through cu_seqlens), each fetched during the one before (about
    8 s of oracle)."""
    cu = [0, 9000, 29001, 34004]
    inp = make_inputs(name="bwdVL", B=1, T=cu[-1], h_qk=2, h_v=8, seed=37, gate="mixed", init_std=0.1,
                      cu_seqlens=cu)
    print(f"\n[bwd/varlen/items] cu={cu}", flush=True)
    d_out, d_fin = _grads(137, inp.v.shape, len(cu) - 1, inp.h_v)
    got = _run(inp, d_out, d_fin)
    _check(inp, d_out, d_fin, got, "varlen/many items")


@pytest.mark.parametrize("config", ["tp8", "tp2", "tp1", "long"])
def test_bwd_full_size(config):
    """The workloads at full size (T = 32768 at the TP8, TP2 and TP1 head
    counts; T = 262144 with an initial state; AutoCP splits every one into
    segments, so the segment maps, the linking pass and the re-run all take
    part): every gradient element against the fp64 backward oracle (about 7 s
    per 2.6e5 head-tokens on 8 host threads: TP8 7 s, TP2 21 s, TP1 14 s,
    long 56 s)."""
    from gated_deltanet_chunked_03_amd.synth import config_inputs
    inp = config_inputs(config)
    print(f"\n[bwd/full/{config}] T={inp.T} h_qk={inp.h_qk} h_v={inp.h_v}", flush=True)
    d_out, d_fin = _grads(177, inp.v.shape, inp.n_seqs, inp.h_v)
    got = _run(inp, d_out, d_fin)
    _check(inp, d_out, d_fin, got, f"full/{config}")


def test_bwd_full_size_fp32_tp8():
    """The TP8 workload with fp32 q, k, v and loss gradient (AutoCP on):
    every gradient element against the oracle at the rounded and at the given
    inputs (two oracle runs, about 14 s)."""
    from gated_deltanet_chunked_03_amd.synth import config_inputs
    inp = config_inputs("tp8", io_dtype="f32")
    print(f"\n[bwd/full/tp8/fp32] T={inp.T} h_qk={inp.h_qk} h_v={inp.h_v}", flush=True)
    d_out, d_fin = _grads(178, inp.v.shape, inp.n_seqs, inp.h_v, io="f32")
    got = _run(inp, d_out, d_fin)
    _check_fp32_inputs(inp, d_out, d_fin, got, "full/tp8/fp32")
