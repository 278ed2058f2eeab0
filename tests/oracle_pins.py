"""Pins for a sequential gated-delta-rule oracle.

Each pin checks an oracle callable ``f(q, k, v, g, beta, scale, S0, cu) -> (o, S_final)``
(shapes as ``oracle.gdn_sequential``) against something fixed outside that oracle:
a hand-worked example, an exact rational brute force of the matrix-product form,
closed forms of special cases, or identities the recurrence must satisfy. The
pins are functions so that the mutation test can run them against oracles with
planted mistakes.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np

from oracle import gdn_exact_fraction

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _unit_rows(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _rand_case(seed, T=7, h_qk=1, h_v=1, d_k=3, d_v=2, s0=True, n_seqs=1):
    r = _rng(seed)
    q = _unit_rows(r.standard_normal((T, h_qk, d_k)))
    k = _unit_rows(r.standard_normal((T, h_qk, d_k)))
    v = r.standard_normal((T, h_v, d_v))
    g = -np.log1p(np.exp(r.standard_normal((T, h_v))))
    beta = 1.0 / (1.0 + np.exp(-r.standard_normal((T, h_v))))
    S0 = r.standard_normal((n_seqs, h_v, d_k, d_v)) * 0.5 if s0 else None
    return q, k, v, g, beta, S0


def pin_hand_example(f):
    """Two tokens worked by hand (tests/golden/hand_example.json)."""
    with open(os.path.join(GOLDEN, "hand_example.json")) as fh:
        ex = json.load(fh)
    q = np.array(ex["q"], float)[:, None, :]
    k = np.array(ex["k"], float)[:, None, :]
    v = np.array(ex["v"], float)[:, None, :]
    g = np.log(np.array(ex["alpha"], float))[:, None]
    b = np.array(ex["beta"], float)[:, None]
    S0 = np.array(ex["S0"], float)[None, None]
    o, S = f(q, k, v, g, b, ex["scale"], S0, None)
    np.testing.assert_allclose(o[:, 0], np.array(ex["o"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(S[0, 0], np.array(ex["S_final"]), rtol=0, atol=1e-12)


def pin_exact_rational(f, seed=0, T=5, d_k=3, d_v=2):
    """Exact rational brute force of S_t = a S (I - b k k^T) + b v k^T, o = S q,
    on small rationals (the gate is rational, its log goes to the oracle)."""
    r = _rng(seed)
    fr = lambda: Fraction(int(r.integers(-4, 5)), int(r.integers(1, 5)))  # noqa: E731
    q = [[fr() for _ in range(d_k)] for _ in range(T)]
    k = [[fr() for _ in range(d_k)] for _ in range(T)]
    v = [[fr() for _ in range(d_v)] for _ in range(T)]
    a = [Fraction(int(r.integers(1, 8)), 8) for _ in range(T)]
    b = [Fraction(int(r.integers(0, 5)), 8) for _ in range(T)]
    S0 = [[fr() for _ in range(d_k)] for _ in range(d_v)]   # recurrent orientation
    scale = Fraction(1, 2)
    o_ex, S_ex = gdn_exact_fraction(q, k, v, a, b, scale, S0)
    F = lambda x: np.array(x, dtype=float)  # noqa: E731
    o, S = f(F(q)[:, None], F(k)[:, None], F(v)[:, None], np.log(F(a))[:, None],
             F(b)[:, None], float(scale), F(S0).T[None, None], None)
    ref_o = F(o_ex)
    np.testing.assert_allclose(o[:, 0], ref_o, rtol=1e-12, atol=1e-12 * np.abs(ref_o).max())
    np.testing.assert_allclose(S[0, 0], F(S_ex).T, rtol=1e-12, atol=1e-12 * np.abs(F(S_ex)).max())


def pin_no_write_no_decay(f, seed=1):
    """beta = 0 and alpha = 1: nothing is written, so o_t = scale S0^T q_t
    (zero when S0 = 0) and the state is unchanged."""
    q, k, v, g, b, S0 = _rand_case(seed, T=9, d_k=4, d_v=3)
    g[:] = 0.0
    b[:] = 0.0
    o, S = f(q, k, v, g, b, 0.7, S0, None)
    np.testing.assert_allclose(o[:, 0], 0.7 * q[:, 0] @ S0[0, 0], atol=1e-13)
    np.testing.assert_allclose(S, S0, atol=1e-13)
    o, S = f(q, k, v, g, b, 0.7, None, None)
    assert np.abs(o).max() == 0.0 and np.abs(S).max() == 0.0


def pin_orthonormal_recall(f, seed=2):
    """beta = 1, alpha = 1, orthonormal keys: after writing (k_s, v_s) the state
    recalls S^T k_s = v_s exactly, for any initial state; a query equal to an
    earlier key reads back scale * v_s."""
    r = _rng(seed)
    d_k, d_v, T = 6, 4, 6
    Qm, _ = np.linalg.qr(r.standard_normal((d_k, d_k)))
    k = Qm.T[:T][:, None, :]                        # rows orthonormal
    v = r.standard_normal((T, 1, d_v))
    src = r.integers(0, T, size=T)
    src = np.minimum(src, np.arange(T))             # query a key already written
    q = k[src]
    g = np.zeros((T, 1))
    b = np.ones((T, 1))
    S0 = r.standard_normal((1, 1, d_k, d_v))
    o, S = f(q, k, v, g, b, 0.5, S0, None)
    np.testing.assert_allclose(o[:, 0], 0.5 * v[src, 0], atol=1e-12)
    np.testing.assert_allclose(k[:, 0] @ S[0, 0], v[:, 0], atol=1e-12)


def pin_delta_recall_any_gate(f, seed=3):
    """beta |k|^2 = 1 makes the updated state predict the written value exactly,
    whatever the gate and the incoming state: S_t^T k_t = v_t (one-token
    sequences with random initial states)."""
    r = _rng(seed)
    n, d_k, d_v = 5, 4, 3
    k = _unit_rows(r.standard_normal((n, 1, d_k)))
    q = _unit_rows(r.standard_normal((n, 1, d_k)))
    v = r.standard_normal((n, 1, d_v))
    g = -r.uniform(0.0, 3.0, size=(n, 1))
    b = np.ones((n, 1))
    S0 = r.standard_normal((n, 1, d_k, d_v))
    _, S = f(q, k, v, g, b, 1.0, S0, np.arange(n + 1))
    for i in range(n):
        np.testing.assert_allclose(k[i, 0] @ S[i, 0], v[i, 0], atol=1e-12)


def pin_gate_closed(f, seed=4):
    """g = -80 (alpha ~ 1e-35): each token sees an empty state, so
    o_t = scale b_t (k_t . q_t) v_t."""
    q, k, v, g, b, S0 = _rand_case(seed, T=8, d_k=5, d_v=3)
    g[:] = -80.0
    o, _ = f(q, k, v, g, b, 0.3, S0, None)
    ref = 0.3 * (b[:, 0] * np.sum(k[:, 0] * q[:, 0], axis=-1))[:, None] * v[:, 0]
    np.testing.assert_allclose(o[:, 0], ref, atol=1e-12)


def pin_single_token(f, seed=5):
    """T = 1: o = scale (a S0^T q + b (k.q)(v - a S0^T k))."""
    q, k, v, g, b, S0 = _rand_case(seed, T=1, d_k=4, d_v=5)
    o, _ = f(q, k, v, g, b, 0.9, S0, None)
    a = math.exp(g[0, 0])
    S = S0[0, 0]
    ref = 0.9 * (a * S.T @ q[0, 0] + b[0, 0] * (k[0, 0] @ q[0, 0]) * (v[0, 0] - a * S.T @ k[0, 0]))
    np.testing.assert_allclose(o[0, 0], ref, atol=1e-13)


def pin_continuation(f, seed=6):
    """Running x1 || x2 equals running x2 from the final state of x1."""
    q, k, v, g, b, S0 = _rand_case(seed, T=11, h_qk=1, h_v=2, d_k=4, d_v=3)
    o, S = f(q, k, v, g, b, 0.5, S0, None)
    c = 4
    o1, S1 = f(q[:c], k[:c], v[:c], g[:c], b[:c], 0.5, S0, None)
    o2, S2 = f(q[c:], k[c:], v[c:], g[c:], b[c:], 0.5, S1, None)
    np.testing.assert_allclose(np.concatenate([o1, o2]), o, atol=1e-12)
    np.testing.assert_allclose(S2, S, atol=1e-12)


def pin_varlen_is_separate(f, seed=7):
    """A packed batch of sequences equals separate runs (each from its own state)."""
    q, k, v, g, b, _ = _rand_case(seed, T=13, h_qk=2, h_v=4, d_k=3, d_v=2, s0=False)
    cu = np.array([0, 5, 5, 13])
    S0 = _rng(seed + 100).standard_normal((3, 4, 3, 2))
    o, S = f(q, k, v, g, b, 1.0, S0, cu)
    for n in range(3):
        a, e = cu[n], cu[n + 1]
        on, Sn = f(q[a:e], k[a:e], v[a:e], g[a:e], b[a:e], 1.0, S0[n:n + 1], None)
        np.testing.assert_allclose(o[a:e], on, atol=1e-12)
        np.testing.assert_allclose(S[n], Sn[0], atol=1e-12)
    np.testing.assert_allclose(S[1], S0[1], atol=0)  # empty sequence passes its state through


def pin_linearity(f, seed=8):
    """For fixed q, k, g, beta the output and state are linear in (v, S0) jointly."""
    q, k, v1, g, b, S1 = _rand_case(seed, T=6, d_k=3, d_v=3)
    _, _, v2, _, _, S2 = _rand_case(seed + 1, T=6, d_k=3, d_v=3)
    oa, Sa = f(q, k, 2.0 * v1 - 3.0 * v2, g, b, 1.0, 2.0 * S1 - 3.0 * S2, None)
    o1, F1 = f(q, k, v1, g, b, 1.0, S1, None)
    o2, F2 = f(q, k, v2, g, b, 1.0, S2, None)
    np.testing.assert_allclose(oa, 2.0 * o1 - 3.0 * o2, atol=1e-11)
    np.testing.assert_allclose(Sa, 2.0 * F1 - 3.0 * F2, atol=1e-11)


def pin_head_grouping(f, seed=9):
    """Value head h reads query/key head floor(h * h_qk / h_v): the grouped run
    equals a run with each value head's query/key copied out explicitly."""
    q, k, v, g, b, _ = _rand_case(seed, T=6, h_qk=2, h_v=6, d_k=3, d_v=2, s0=False)
    o, S = f(q, k, v, g, b, 1.0, None, None)
    idx = np.array([h * 2 // 6 for h in range(6)])
    assert list(idx) == [0, 0, 0, 1, 1, 1]
    o2, S2 = f(q[:, idx], k[:, idx], v, g, b, 1.0, None, None)
    np.testing.assert_allclose(o, o2, atol=1e-13)
    np.testing.assert_allclose(S, S2, atol=1e-13)


ALL_PINS = [pin_hand_example, pin_exact_rational, pin_no_write_no_decay,
            pin_orthonormal_recall, pin_delta_recall_any_gate, pin_gate_closed,
            pin_single_token, pin_continuation, pin_varlen_is_separate,
            pin_linearity, pin_head_grouping]
