"""The fp64 chunked (WY) model and its context-parallel variants against the
sequential oracle and the identities that define them (CPU only)."""
from __future__ import annotations

import math

import numpy as np
import pytest

from oracle import chunk_model as cm
from oracle import gdn_sequential
from gated_deltanet_chunked_03_amd.synth import make_inputs


def _case(T, h_qk=1, h_v=2, d=16, seed=0, gate="mixed", init_std=0.2, cu=None, **kw):
    inp = make_inputs(1, T, h_qk, h_v, d_k=d, d_v=d, seed=seed, gate=gate, init_std=init_std,
                      cu_seqlens=cu, **kw)
    q, k, v, g, b = inp.flat()
    return inp, q, k, v, g, b


def test_chunk_prep_defining_equations():
    """A strictly lower, T unit lower triangular, (I + A) W = diag(b e^gamma) K and
    (I + A) U = diag(b) V: the WY factors solve the chunk's triangular system."""
    r = np.random.default_rng(0)
    c, d = 64, 8
    k = r.standard_normal((c, d)); k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = r.standard_normal((c, d))
    g = -r.uniform(0, 0.5, c)
    b = r.uniform(0, 1, c)
    gam, A, T, W, U = cm.chunk_prep(k, v, g, b)
    np.testing.assert_allclose(gam, np.cumsum(g))
    assert np.all(np.triu(A) == 0)
    np.testing.assert_allclose(np.diag(T), 1.0)
    assert np.abs(np.triu(T, 1)).max() < 1e-14
    I = np.eye(c)
    np.testing.assert_allclose((I + A) @ W, (b * np.exp(gam))[:, None] * k, atol=1e-12)
    np.testing.assert_allclose((I + A) @ U, b[:, None] * v, atol=1e-12)
    # one entry of A by its definition
    np.testing.assert_allclose(A[5, 2], b[5] * math.exp(gam[5] - gam[2]) * (k[5] @ k[2]))


def test_chunk_affine_matches_forward_step():
    r = np.random.default_rng(1)
    c, d = 40, 8
    k = r.standard_normal((c, d)) / 3
    q = r.standard_normal((c, d))
    v = r.standard_normal((c, d))
    g = -r.uniform(0, 0.3, c)
    b = r.uniform(0, 1, c)
    gam, _, _, W, U = cm.chunk_prep(k, v, g, b)
    M, H = cm.chunk_affine(k, gam, W, U)
    S = r.standard_normal((d, d))
    _, S1, _ = cm.chunk_forward(S, q, k, gam, W, U, 1.0)
    np.testing.assert_allclose(M @ S + H, S1, atol=1e-12)


@pytest.mark.parametrize("T,cu", [(64, None), (200, None), (517, None),
                                  (300, [0, 1, 64, 65, 300])])
def test_chunked_equals_sequential(T, cu):
    inp, q, k, v, g, b = _case(T, h_qk=1, h_v=2, seed=T, cu=cu,
                               init_std=None if cu else 0.2)
    S0 = inp.initial_state
    o_ref, S_ref, _ = gdn_sequential(q, k, v, g, b, inp.scale, S0, cu)
    o, S, _ = cm.chunked_forward(q, k, v, g, b, inp.scale, S0, cu, mode="off")
    assert np.abs(o - o_ref).max() <= 1e-12 * max(1.0, np.abs(o_ref).max())
    assert np.abs(S - S_ref).max() <= 1e-12 * max(1.0, np.abs(S_ref).max())


@pytest.mark.parametrize("L", [1, 2, 3, 7, 100])
def test_exact_cp_equals_sequential(L):
    """Exact context parallelism: the segment initial states composed from the
    chunk maps are the true states at the boundaries, so outputs agree."""
    T = 64 * 9 + 17
    inp, q, k, v, g, b = _case(T, h_qk=1, h_v=2, seed=10 + L, gate="mixed")
    o_ref, S_ref, snaps = gdn_sequential(q, k, v, g, b, inp.scale, inp.initial_state,
                                         snap_stride=64 * L, n_snap=12)
    o, S, info = cm.chunked_forward(q, k, v, g, b, inp.scale, inp.initial_state, L=L,
                                    mode="exact")
    assert np.abs(o - o_ref).max() <= 1e-11 * np.abs(o_ref).max()
    assert np.abs(S - S_ref).max() <= 1e-11 * np.abs(S_ref).max()
    for h in range(2):
        for s, S0s in enumerate(info["S0"][0][h]):
            np.testing.assert_allclose(S0s, snaps[0, h, s], atol=1e-11 * np.abs(snaps).max())


def test_warmup_error_within_contraction_bound():
    """Warm-up from zero over the w chunks before a boundary differs from the
    true state by at most exp(sum of g over the window) * |S at window start|_F
    (each token map a (I - b k k^T) has spectral norm <= a when b |k|^2 <= 2)."""
    T, L, w = 64 * 12, 3, 2
    inp, q, k, v, g, b = _case(T, h_qk=1, h_v=1, seed=5, gate="slow", init_std=0.5)
    o_ref, _, snaps = gdn_sequential(q, k, v, g, b, inp.scale, inp.initial_state,
                                     snap_stride=64, n_snap=13)
    _, _, info = cm.chunked_forward(q, k, v, g, b, inp.scale, inp.initial_state, L=L,
                                    mode="warmup", w=w)
    S0s = info["S0"][0][0]
    checked = 0
    for s in range(1, len(S0s)):
        a = s * L
        lo = max(a - w, 0)
        err = np.linalg.norm(S0s[s] - snaps[0, 0, a])
        if lo == 0:
            assert err < 1e-12
            continue
        bound = math.exp(float(np.sum(g[lo * 64:a * 64, 0], dtype=np.float64))) * \
            np.linalg.norm(snaps[0, 0, lo])
        assert err <= bound * (1 + 1e-9) + 1e-12
        assert err > 0.0
        checked += 1
    assert checked >= 2


def test_adaptive_warmup_window():
    """The warm-up window is the shortest run of whole chunks before the
    boundary (at most w) whose log-decay reaches ln(eps); the w chunks if none
    does; [0, a) when the w-chunk window would reach the sequence start."""
    eps, w = 1e-4, 6
    g = np.zeros(64 * 16)
    g[64 * 9:64 * 10] = -83.0 / 64          # chunk 9 alone decays far below eps
    assert cm.warmup_window(10, w, g, eps) == (9, 10)
    g[:] = 0.0
    g[64 * 7:64 * 10] = -4.0 / 64           # -4 per chunk: three chunks needed (-12 <= ln 1e-4)
    assert cm.warmup_window(10, w, g, eps) == (7, 10)
    g[:] = -1e-4                            # slow decay: no run of <= w chunks qualifies
    assert cm.warmup_window(10, w, g, eps) == (4, 10)
    assert cm.warmup_window(10, w) == (4, 10)
    assert cm.warmup_window(5, w, g, eps) == (0, 5)
    assert cm.warmup_window(6, w, g, eps) == (0, 6)


def test_adaptive_warmup_error_within_bound():
    """With fast-decay gates the adaptive window is one chunk, and the state it
    misses is bounded by exp(sum g over that chunk) |S at the window start|."""
    T, L, w, eps = 64 * 12, 3, 6, 1e-4
    inp, q, k, v, g, b = _case(T, h_qk=1, h_v=1, seed=7, gate="fast", init_std=0.5)
    _, _, snaps = gdn_sequential(q, k, v, g, b, inp.scale, inp.initial_state, snap_stride=64, n_snap=13)
    _, _, info = cm.chunked_forward(q, k, v, g, b, inp.scale, inp.initial_state, L=L, mode="warmup",
                                    w=w, eps=eps)
    S0s = info["S0"][0][0]
    for s in range(1, len(S0s)):
        a = s * L
        lo, hi = cm.warmup_window(a, w, g[:, 0], eps)
        assert hi == a and (lo == 0 or lo == a - 1)
        err = np.linalg.norm(S0s[s] - snaps[0, 0, a])
        if lo == 0:
            assert err < 1e-12
            continue
        bound = math.exp(float(np.sum(g[lo * 64:a * 64, 0], dtype=np.float64))) * np.linalg.norm(snaps[0, 0, lo])
        # fp64 rounding of the two evaluation orders on top of the bound
        assert err <= bound * (1 + 1e-9) + 1e-12 * np.linalg.norm(snaps[0, 0, a])
        assert bound <= eps * np.linalg.norm(snaps[0, 0, lo])


def test_warmup_exact_when_window_reaches_start():
    T = 64 * 5
    inp, q, k, v, g, b = _case(T, h_qk=1, h_v=2, seed=6, gate="slow")
    o_ref, S_ref, _ = gdn_sequential(q, k, v, g, b, inp.scale, inp.initial_state)
    o, S, _ = cm.chunked_forward(q, k, v, g, b, inp.scale, inp.initial_state, L=2,
                                 mode="warmup", w=6)
    assert np.abs(o - o_ref).max() <= 1e-11 * np.abs(o_ref).max()


def test_fast_heads_warm_up_and_meet_state_error_budget():
    """Gate-driven path choice on the synthetic mix: fast-decay heads take the
    warm-up path, slow heads the exact path, and the warm-up states are within
    1e-3 relative Frobenius error of the true boundary states."""
    T, L = 64 * 24, 8
    inp, q, k, v, g, b = _case(T, h_qk=2, h_v=8, seed=2, gate="mixed", d=16)
    o_ref, _, snaps = gdn_sequential(q, k, v, g, b, inp.scale, None, snap_stride=64 * L,
                                     n_snap=4)
    o, _, info = cm.chunked_forward(q, k, v, g, b, inp.scale, None, L=L, mode="auto")
    for h, cls in enumerate(inp.head_class):
        assert info["path"][0][h] == ("warmup" if cls == "fast" else "exact")
        for s, S0s in enumerate(info["S0"][0][h][1:], start=1):
            ref = snaps[0, h, s]
            assert np.linalg.norm(S0s - ref) <= 1e-3 * np.linalg.norm(ref)
    assert np.abs(o - o_ref).sum() <= 1e-6 * np.abs(o_ref).sum()


def test_prep_all_layout_and_padding():
    cu = [0, 70, 70, 200]
    inp, q, k, v, g, b = _case(200, h_qk=1, h_v=2, seed=7, cu=cu, init_std=None)
    G, W, U = cm.prep_all(k, v, g, b, h_v=2, cu_seqlens=cu)
    assert G.shape[0] == 2 + 0 + 3
    # second chunk of sequence 0 holds 6 tokens; rows past them are padding
    gam, _, _, W1, U1 = cm.chunk_prep(k[64:70, 0], v[64:70, 1], g[64:70, 1], b[64:70, 1])
    np.testing.assert_allclose(G[1, 1, :6], gam)
    np.testing.assert_allclose(G[1, 1, 6:], gam[-1])
    np.testing.assert_allclose(W[1, 1, :6], W1)
    assert np.all(W[1, 1, 6:] == 0) and np.all(U[1, 1, 6:] == 0)


def _switch_gates(N, switch_chunk, slow=-2e-4, fast=-0.4, fast_first=False):
    """One head whose gates switch regime at a chunk: slow decay before it
    (no run of <= 6 chunks decays below 1e-4), fast after it (one chunk does);
    or the reverse with fast_first."""
    a, b = (fast, slow) if fast_first else (slow, fast)
    g = np.full(64 * N, a)
    g[64 * switch_chunk:] = b
    return g


def test_boundary_rule_regime_switch_and_windows():
    """The per-boundary rule, pinned by gates whose chunk sums are known in
    closed form: a head that switches from slow to fast decay mid-sequence is
    exact before the switch and warms up (one chunk) after it (summary: mixed);
    constant decays of ln(eps) / (j - 1/2) per chunk give windows of exactly j
    chunks for j = 2..5; boundaries within w chunks of the start are 'start'."""
    eps, w, L, N = 1e-4, 6, 4, 40
    g = _switch_gates(N, 20)
    kinds = [cm.boundary_rule(g, a, w, eps) for a in range(L, N, L)]
    # a = 4: window reaches the start; 8..20: the chunks before a are all slow
    # (6 chunks sum to -0.077 > ln 1e-4); 24..36: chunk a - 1 is fast (-25.6)
    expect = [("start", 4)] + [("exact", 0)] * 4 + [("warmup", 1)] * 4
    assert kinds == expect
    assert cm.boundary_summary(kinds) == 2
    assert cm.boundary_summary([("start", 4), ("warmup", 1)]) == 1
    assert cm.boundary_summary([("start", 4), ("exact", 0)]) == 0
    assert cm.boundary_summary([("start", 4)]) == 3
    for j in range(2, 6):
        per_chunk = math.log(eps) / (j - 0.5)
        gj = np.full(64 * 20, per_chunk / 64)
        assert cm.boundary_rule(gj, 12, w, eps) == ("warmup", j), j
    # a run that never decays far enough stays exact even at the window's end
    assert cm.boundary_rule(np.full(64 * 20, math.log(eps) / (6.5 * 64)), 12, w, eps) == ("exact", 0)


@pytest.mark.parametrize("switch,fast_first", [(20, False), (9, False), (14, True)])
def test_boundary_mode_states(switch, fast_first):
    """'boundary' mode against the sequential oracle's states: exact boundaries
    (the previous segment's map applied to the previous boundary's state, even
    when that one was warmed up) to fp64 accuracy on top of the inherited
    warm-up error; warm-up boundaries within the contraction bound
    exp(sum g over the window) |S at the window start|; 'start' boundaries
    exact."""
    T, L, w, eps = 64 * 32, 4, 6, 1e-4
    inp, q, k, v, g, b = _case(T, h_qk=1, h_v=1, seed=17, gate="plain", init_std=0.5)
    g[:, 0] = _switch_gates(32, switch, fast_first=fast_first).astype(np.float32)
    _, _, snaps = gdn_sequential(q, k, v, g, b, inp.scale, inp.initial_state, snap_stride=64, n_snap=33)
    o, fin, info = cm.chunked_forward(q, k, v, g, b, inp.scale, inp.initial_state, L=L, mode="boundary",
                                      w=w, eps=eps)
    S0s, kinds = info["S0"][0][0], info["boundary"][0][0]
    assert info["path"][0][0] == 2
    prev_err = 0.0
    for s in range(1, len(S0s)):
        a = s * L
        kind, j = kinds[s - 1]
        err = np.linalg.norm(S0s[s] - snaps[0, 0, a])
        if kind == "start":
            assert err < 1e-10 * np.linalg.norm(snaps[0, 0, a])
        elif kind == "warmup":
            bound = math.exp(float(np.sum(g[(a - j) * 64:a * 64, 0], dtype=np.float64))) * \
                np.linalg.norm(snaps[0, 0, a - j])
            assert 0.0 < err <= bound * (1 + 1e-9) + 1e-12
        else:
            # the map is exact; an error inherited from the previous boundary
            # only contracts through the segment (|M|_2 <= 1 here)
            assert err <= prev_err * (1 + 1e-9) + 1e-10 * np.linalg.norm(snaps[0, 0, a])
        prev_err = err
    # the reversed switch has exact boundaries after warmed-up ones
    if fast_first:
        assert ("exact", 0) in kinds and kinds.index(("exact", 0)) > kinds.index(("warmup", 1))
