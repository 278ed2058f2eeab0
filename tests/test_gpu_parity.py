"""HIP path against the fp64 oracle, element by element, through the C ABI.

Sizes here span several chunks, a ragged final chunk and several segments;
the full-size workloads are in test_gpu_configs.py.
"""
from __future__ import annotations

import numpy as np
import pytest

from gated_deltanet_chunked_03_amd.synth import make_inputs
from gpu_util import BOUNDARY_TOL, STATE_MAX_TOL, STATE_MEAN_TOL, assert_within_tolerance, errors, oracle_run, to_device
from oracle import chunk_model

pytestmark = pytest.mark.gpu


def _gdn():
    import gated_deltanet_chunked_03_amd as gdn
    return gdn


def _run(inp, **kw):
    import torch
    gdn = _gdn()
    d = to_device(inp)
    res = gdn.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], scale=inp.scale,
                  initial_state=d["initial_state"], cu_seqlens=inp.cu_seqlens, **kw)
    torch.cuda.synchronize()
    return res


def _o_np(o, inp):
    return o.float().cpu().numpy().reshape(inp.B * inp.T, inp.h_v, -1)


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_chunk_prep_matches_model(io):
    """gamma, W, U of the chunk-prep kernel against the fp64 chunk model
    (ragged final chunk, grouped heads)."""
    import torch
    inp = make_inputs(1, 64 * 3 + 21, 2, 4, seed=21, gate="mixed", io_dtype=io)
    d = to_device(inp)
    gam, W, U = _gdn().chunk_prep(d["k"], d["v"], d["g"], d["beta"])
    torch.cuda.synchronize()
    q, k, v, g, b = inp.flat()
    G0, W0, U0 = chunk_model.prep_all(k, v, g, b, h_v=inp.h_v)
    print(f"[chunk_prep {io}] shapes {tuple(W.shape)}", flush=True)
    assert errors(gam.cpu().numpy(), G0)[0] < 1e-5
    # Each MFMA operand that is not an exact bf16 input is a hi + lo bf16 pair
    # (relative representation error <= 2^-16); a product of two such operands
    # with fp32 accumulation is good to about 3 * 2^-16 = 4.6e-5 per term.
    for name, x, ref in (("W", W, W0), ("U", U, U0)):
        mx, mean = errors(x.cpu().numpy(), ref)
        print(f"  {name}: max-rel {mx:.2e} mean-rel {mean:.2e}")
        assert mx < 1e-4 and mean < 3e-5, name


@pytest.mark.parametrize("io,T,h_qk,h_v", [("bf16", 64 * 5 + 13, 2, 4), ("f32", 512, 1, 1),
                                           ("bf16", 64, 1, 3), ("bf16", 1, 1, 1)])
def test_fwd_single_segment(io, T, h_qk, h_v):
    inp = make_inputs(1, T, h_qk, h_v, seed=T + h_v, gate="mixed" if h_v > 1 else "plain",
                      io_dtype=io, init_std=0.1)
    o, S = _run(inp, cp_mode="off")
    o_ref, S_ref, _ = oracle_run(inp)
    mx, mean = assert_within_tolerance(_o_np(o, inp), o_ref)
    smx, smean = assert_within_tolerance(S.cpu().numpy(), S_ref, "final_state", STATE_MAX_TOL, STATE_MEAN_TOL)
    print(f"[fwd off {io} T={T} {h_qk}/{h_v}] o {mx:.2e}/{mean:.2e} S {smx:.2e}/{smean:.2e}")


@pytest.mark.parametrize("io,layout", [("bf16", 1), ("bf16", 2), ("f32", 0)])
@pytest.mark.parametrize("mode", ["exact", "warmup", "auto"])
def test_fwd_context_parallel(mode, io, layout):
    """Segments of L chunks with exact or warm-up boundary states: outputs
    within tolerance and the segment initial states close to the true states
    (exact: to fp32 accuracy; warm-up on fast heads: <= 1e-3 relative), for
    bf16 inputs in both boundary preprocessing layouts (H and M of an exact
    boundary in one workgroup or in two) and for fp32 inputs."""
    import torch
    T, L = 64 * 40 + 5, 4
    inp = make_inputs(1, T, 2, 8, seed=30, gate="mixed", init_std=0.05, io_dtype=io)
    o, S, info = _run(inp, cp_mode=mode, n_cu=32, lam=0.6, debug=True, cp_layout=layout)
    plan = info["plan"]
    print(f"[cp {mode} {io} layout {layout}] plan L={plan['L']} P={plan['P_max']} segs={plan['n_segments']}")
    assert plan["cp_on"] == 1 and plan["L"] == L and plan["cp_layout"] == layout
    o_ref, S_ref, snaps = oracle_run(inp, snap_stride=64 * L, n_snap=plan["P_max"])
    seg = info["seg_state"].cpu().numpy()
    path = info["path"].cpu().numpy()
    print(f"  path {path.tolist()} classes {inp.head_class}")
    for h, cls in enumerate(inp.head_class):
        rel = [np.linalg.norm(seg[s, h] - snaps[0, h, s]) / np.linalg.norm(snaps[0, h, s])
               for s in range(1, plan["P_max"])]
        print(f"  head {h} ({cls}) boundary state rel err max {max(rel):.2e}")
        if mode == "exact" or (mode == "auto" and cls != "fast"):
            assert max(rel) < BOUNDARY_TOL
        if mode == "auto":
            assert path[0, h] == (1 if cls == "fast" else 0)
        if cls == "fast":
            assert max(rel) < BOUNDARY_TOL
    if mode != "warmup":  # forced warm-up on slow heads is approximate by design
        assert_within_tolerance(_o_np(o, inp), o_ref)
        assert_within_tolerance(S.cpu().numpy(), S_ref, "final_state", STATE_MAX_TOL, STATE_MEAN_TOL)
    else:
        fast = [h for h, c in enumerate(inp.head_class) if c == "fast"]
        assert_within_tolerance(_o_np(o, inp)[:, fast], o_ref[:, fast])


@pytest.mark.parametrize("layout", [1, 2])
def test_varlen_with_initial_state(layout):
    """Packed sequences (including an empty one and a one-token one) with
    per-sequence initial states equal separate oracle runs (both boundary
    preprocessing layouts)."""
    cu = [0, 700, 700, 701, 64 * 20 + 3, 64 * 20 + 3 + 130]
    T = cu[-1]
    inp = make_inputs(1, T, 1, 4, seed=40, gate="mixed", cu_seqlens=cu, init_std=0.1)
    for mode in ("off", "auto", "exact"):
        o, S = _run(inp, cp_mode=mode, n_cu=64, lam=0.5, warmup_chunks=2, cp_layout=layout)
        o_ref, S_ref, _ = oracle_run(inp)
        mx, mean = assert_within_tolerance(_o_np(o, inp), o_ref)
        assert_within_tolerance(S.cpu().numpy(), S_ref, "final_state", STATE_MAX_TOL, STATE_MEAN_TOL)
        np.testing.assert_allclose(S.cpu().numpy()[1], inp.initial_state[1], rtol=0, atol=0)
        print(f"[varlen {mode} layout {layout}] o {mx:.2e}/{mean:.2e}")


def test_deterministic_rerun():
    import torch
    inp = make_inputs(1, 64 * 24, 2, 8, seed=50, gate="mixed")
    o1, S1 = _run(inp, cp_mode="auto", n_cu=256)
    o2, S2 = _run(inp, cp_mode="auto", n_cu=256)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_gate_closed_and_no_write_special_cases():
    """g = -80 (state erased every token): o_t = scale beta_t (k_t.q_t) v_t;
    beta = 0 and g = 0: o_t = scale S0^T q_t."""
    import torch
    gdn = _gdn()
    inp = make_inputs(1, 64 * 3 + 7, 1, 2, seed=60, init_std=0.2)
    d = to_device(inp)
    g = torch.full_like(d["g"], -80.0)
    o, _ = gdn.fwd(d["q"], d["k"], d["v"], g, d["beta"], scale=0.5, initial_state=d["initial_state"])
    q, k, v, _, b = inp.flat()
    qk = np.sum(q.astype(np.float64) * k, axis=-1)                  # [T, 1]
    ref = 0.5 * (b * qk)[..., None] * v
    assert_within_tolerance(o.float().cpu().numpy().reshape(ref.shape), ref)
    o, S = gdn.fwd(d["q"], d["k"], d["v"], torch.zeros_like(d["g"]), torch.zeros_like(d["beta"]),
                   scale=0.5, initial_state=d["initial_state"])
    torch.cuda.synchronize()
    ref = 0.5 * np.einsum("tk,hkv->thv", q[:, 0].astype(np.float64), inp.initial_state[0])
    assert_within_tolerance(o.float().cpu().numpy().reshape(ref.shape), ref)
    np.testing.assert_array_equal(S.cpu().numpy(), inp.initial_state)


def test_empty_inputs_pass_the_state_through():
    """No tokens (T = 0, and packed sequences that are all empty): nothing to
    write, and the final state is the initial state (zeros without one)."""
    import torch
    gdn = _gdn()
    dev = torch.device("cuda")
    S0 = torch.randn(2, 3, 128, 128, device=dev)
    for cu in (None, [0, 0, 0]):
        B = 2 if cu is None else 1
        q = torch.zeros(B, 0, 1, 128, dtype=torch.bfloat16, device=dev)
        v = torch.zeros(B, 0, 3, 128, dtype=torch.bfloat16, device=dev)
        g = torch.zeros(B, 0, 3, device=dev)
        for mode in ("off", "auto"):
            o, S = gdn.fwd(q, q, v, g, g, scale=0.1, initial_state=S0, cu_seqlens=cu, cp_mode=mode)
            o2, S2 = gdn.fwd(q, q, v, g, g, scale=0.1, cu_seqlens=cu, cp_mode=mode)
            torch.cuda.synchronize()
            assert o.numel() == 0 and torch.equal(S, S0) and torch.count_nonzero(S2) == 0


@pytest.mark.parametrize("mode,io", [("exact", "bf16"), ("auto", "bf16"), ("auto", "f32")])
def test_grouped_combine(mode, io):
    """Many segments per sequence (long boundary chains in the combine; the
    planner also groups them, which the backward's forward re-run uses): two
    packed sequences of different lengths, an initial state, a ragged tail,
    exact and warm-up boundaries. Every boundary state against the oracle's
    state there; outputs at the stated tolerance."""
    cu = [0, 64 * 129 + 37, 64 * 129 + 37 + 64 * 70 + 5]
    inp = make_inputs(1, cu[-1], 2, 4, seed=61, gate="mixed", cu_seqlens=cu, init_std=0.05, io_dtype=io)
    o, S, info = _run(inp, cp_mode=mode, n_cu=256, debug=True)
    plan = info["plan"]
    print(f"\n[grouped {mode} {io}] plan L={plan['L']} P={plan['P_max']} G={plan['combine_group']} "
          f"J={plan['combine_groups']}", flush=True)
    assert plan["cp_on"] == 1 and plan["combine_group"] > 0 and plan["combine_groups"] >= 3
    L = plan["L"]
    o_ref, S_ref, snaps = oracle_run(inp, snap_stride=64 * L, n_snap=plan["P_max"])
    assert_within_tolerance(_o_np(o, inp), o_ref)
    assert_within_tolerance(S.cpu().numpy(), S_ref, "final_state", STATE_MAX_TOL, STATE_MEAN_TOL)
    seg = info["seg_state"].cpu().numpy()
    path = info["path"].cpu().numpy()
    base = 0
    for n in range(inp.n_seqs):
        n_ch = -(-(cu[n + 1] - cu[n]) // 64)
        P = -(-n_ch // L)
        for h, cls in enumerate(inp.head_class):
            rel = [np.linalg.norm(seg[base + s, h] - snaps[n, h, s]) / np.linalg.norm(snaps[n, h, s])
                   for s in range(1, P)]
            print(f"  seq {n} head {h} ({cls}, path {path[n, h]}) boundary state rel err max {max(rel):.2e}")
            if mode == "exact" or cls != "fast":
                assert max(rel) < BOUNDARY_TOL, (n, h)
            else:
                assert max(rel) < BOUNDARY_TOL, (n, h)
        base += P


def test_calibrate_lambda_picks_a_candidate():
    """gdn_calibrate_lambda times every candidate and returns one of them; the
    forward with it matches the oracle like any other plan."""
    import torch
    import gated_deltanet_chunked_03_amd as gdn
    inp = make_inputs(name="calib", B=1, T=64 * 40, h_qk=2, h_v=4, seed=41, gate="mixed")
    d = to_device(inp)
    lams = (0.5, 1.0, 2.0)
    print("\n[calibrate] T=2560 h_v=4 on 16 CUs", flush=True)
    best, ms = gdn.calibrate_lambda(d["q"], d["k"], d["v"], d["g"], d["beta"], lambdas=lams, reps=2,
                                    scale=inp.scale, n_cu=16)
    print(f"[calibrate] best {best}, ms {ms}", flush=True)
    assert best in lams and all(x > 0 for x in ms.values())
    assert ms[best] == min(ms.values())
    o, _ = gdn.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], scale=inp.scale, lam=best, n_cu=16)
    torch.cuda.synchronize()
    o_ref, _, _ = oracle_run(inp)
    assert_within_tolerance(o.float().cpu().numpy().reshape(o_ref.shape), o_ref, "o")


@pytest.mark.parametrize("N,n_cu,lam,grouped", [(49, 32, 0.6, False), (193, 256, 1.0, True)],
                         ids=["chain", "grouped-combine"])
def test_per_boundary_rule_switch_heads_and_windows(N, n_cu, lam, grouped):
    """AUTO decides per boundary: a head whose gates switch from slow to fast
    decay mid-sequence (exact, then warm-up: mixed), one switching the other
    way (exact boundaries chained onto warmed-up ones), and constant decays
    that need warm-up windows of exactly 2, 3, 4 and 5 chunks. With a noise
    floor of 0.05 a window one chunk too short or too long moves the boundary
    state by percents, so every boundary state is compared with the fp64
    chunk model's per-boundary reading of the same inputs (same windows, same
    chaining), and the per-head path codes with the model's. The longer case
    has enough boundaries for the grouped combine, whose composed group maps
    then hold warm-up boundaries between exact ones."""
    import math
    eps, w = 0.05, 6
    T = 64 * (N - 1) + 7
    inp = make_inputs(1, T, 1, 6, seed=71, gate="plain", init_std=0.1)
    g = inp.g
    g[0, :, 0] = -2e-4
    g[0, 64 * (N // 2):, 0] = -0.4            # slow -> fast mid-sequence
    g[0, :, 1] = -0.4
    g[0, 64 * (N * 2 // 5):, 1] = -2e-4       # fast -> slow
    for h, j in zip(range(2, 6), range(2, 6)):
        g[0, :, h] = math.log(eps) / (64 * (j - 0.5))
    o, S, info = _run(inp, cp_mode="auto", n_cu=n_cu, lam=lam, warmup_chunks=w, noise_floor=eps, debug=True)
    plan = info["plan"]
    L = plan["L"]
    print(f"\n[per-boundary] plan L={L} P={plan['P_max']} combine G={plan['combine_group']}", flush=True)
    assert plan["cp_on"] == 1 and (plan["combine_group"] > 0) == grouped
    if not grouped:
        assert L == 4
    q, k, v, gg, b = inp.flat()
    o_m, S_m, minfo = chunk_model.chunked_forward(q, k, v, gg, b, inp.scale, inp.initial_state, L=L,
                                                  mode="boundary", w=w, eps=eps)
    seg = info["seg_state"].cpu().numpy()
    path = info["path"].cpu().numpy()
    for h in range(inp.h_v):
        kinds = minfo["boundary"][0][h]
        rel = [np.linalg.norm(seg[s, h] - minfo["S0"][0][h][s]) / np.linalg.norm(minfo["S0"][0][h][s])
               for s in range(1, plan["P_max"])]
        print(f"  head {h}: path {path[0, h]} (model {minfo['path'][0][h]}) "
              f"windows {sorted(set(j for kk, j in kinds if kk == 'warmup'))} max rel {max(rel):.2e}")
        assert path[0, h] == minfo["path"][0][h], h
        assert max(rel) < BOUNDARY_TOL, h
    assert [minfo["path"][0][h] for h in range(6)] == [2, 2, 1, 1, 1, 1]
    for h, j in zip(range(2, 6), range(2, 6)):
        assert {jj for kk, jj in minfo["boundary"][0][h] if kk == "warmup"} == {j}
    assert_within_tolerance(_o_np(o, inp), o_m)
    assert_within_tolerance(S.cpu().numpy(), S_m, "final_state", STATE_MAX_TOL, STATE_MEAN_TOL)


@pytest.mark.parametrize("dv_split", [1, 2, 4])
def test_fwd_column_split(dv_split):
    """The forward with d_v in 1, 2 or 4 column blocks (one workgroup per
    (sequence, head, block), no segments): outputs and final states against
    the oracle; two sequences, a ragged tail, grouped heads, an initial state."""
    cu = [0, 64 * 9 + 17, 64 * 9 + 17 + 64 * 4]
    inp = make_inputs(1, cu[-1], 2, 4, seed=81, gate="mixed", cu_seqlens=cu, init_std=0.1)
    o, S, info = _run(inp, cp_mode="auto", n_cu=16, dv_split=dv_split, debug=True)
    plan = info["plan"]
    print(f"\n[dv_split {dv_split}] plan cp_on={plan['cp_on']} dv_split={plan['dv_split']}", flush=True)
    assert plan["cp_on"] == 0 and plan["dv_split"] == dv_split
    o_ref, S_ref, _ = oracle_run(inp)
    mx, mean = assert_within_tolerance(_o_np(o, inp), o_ref)
    smx, smean = assert_within_tolerance(S.cpu().numpy(), S_ref, "final_state", STATE_MAX_TOL, STATE_MEAN_TOL)
    print(f"  o {mx:.2e}/{mean:.2e} S {smx:.2e}/{smean:.2e}")
