"""Pins of the fp64 backward oracle (CPU only).

The gradients are pinned to things other than their own derivation:
  - central finite differences of the forward oracle, for every input element
    (q, k, v, g, beta, initial state) on tiny inputs with a GQA head group and
    two packed sequences, through a random linear loss on the outputs and the
    final states;
  - a closed form when beta = 0 (no writes: S_t = exp(g_1 + ... + g_t) S_0);
  - every planted slip in a copy of the reverse pass trips the
    finite-difference pin.
The C and numpy forms are also compared with each other on a larger case.
"""
from __future__ import annotations

import numpy as np
import pytest

from oracle import gdn_sequential, gdn_sequential_bwd, gdn_sequential_bwd_np

FORMS = {"c": gdn_sequential_bwd, "numpy": gdn_sequential_bwd_np}


def _case(seed, T=9, h_qk=1, h_v=2, d_k=3, d_v=2, cu=(0, 4, 9), zero_beta=False):
    r = np.random.default_rng(seed)
    q = r.standard_normal((T, h_qk, d_k))
    k = r.standard_normal((T, h_qk, d_k))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((T, h_v, d_v))
    g = -r.uniform(0.05, 1.0, (T, h_v))
    b = np.zeros((T, h_v)) if zero_beta else r.uniform(0.1, 0.9, (T, h_v))
    n = len(cu) - 1
    s0 = r.standard_normal((n, h_v, d_k, d_v))
    do = r.standard_normal((T, h_v, d_v))
    dfin = r.standard_normal((n, h_v, d_k, d_v))
    return dict(q=q, k=k, v=v, g=g, beta=b, s0=s0, do=do, dfin=dfin, cu=list(cu), scale=0.7)


def _loss(c, **over):
    x = dict(c, **over)
    o, fin, _ = gdn_sequential(x["q"], x["k"], x["v"], x["g"], x["beta"], x["scale"], x["s0"], x["cu"])
    return float(np.sum(o * c["do"]) + np.sum(fin * c["dfin"]))


def _fd(c, name, eps=1e-6):
    base = c[name]
    grad = np.zeros_like(base)
    for idx in np.ndindex(base.shape):
        xp = base.copy()
        xm = base.copy()
        xp[idx] += eps
        xm[idx] -= eps
        grad[idx] = (_loss(c, **{name: xp}) - _loss(c, **{name: xm})) / (2 * eps)
    return grad


def _grads(f, c):
    return f(c["q"], c["k"], c["v"], c["g"], c["beta"], c["scale"], c["do"], c["s0"], c["dfin"], c["cu"])


KEYS = {"q": "dq", "k": "dk", "v": "dv", "g": "dg", "beta": "dbeta", "s0": "d_initial"}


def pin_finite_differences(f, seed=0):
    c = _case(seed)
    got = _grads(f, c)
    for name, key in KEYS.items():
        ref = _fd(c, name)
        err = np.abs(got[key] - ref).max()
        assert err <= 1e-7 * max(1.0, np.abs(ref).max()), f"{key}: finite-difference mismatch {err:.2e}"


def pin_no_write_closed_form(f, seed=1):
    """beta = 0: S_t = A_t S_0 with A_t = exp(g_1 + ... + g_t) (per sequence and
    head), o_t = scale A_t S_0^T q_t, so dv = dk = 0, dq_t = scale A_t S_0 do_t,
    dS_0 = scale sum_t A_t q_t do_t^T + A_T dS_final,
    dg_t = sum_{s >= t} scale A_s q_s^T S_0 do_s + A_T <dS_final, S_0>, and
    dbeta_t = (G_t^T k_t) . (v_t - A_t S_0^T k_t) with G_t the loss gradient of
    S_t: scale sum_{s >= t} (A_s / A_t) q_s do_s^T + (A_T / A_t) dS_final."""
    c = _case(seed, zero_beta=True)
    got = _grads(f, c)
    assert np.abs(got["dv"]).max() == 0 and np.abs(got["dk"]).max() == 0
    q, k, v, g, do, s0, dfin, cu, sc = (c[x] for x in ("q", "k", "v", "g", "do", "s0", "dfin", "cu", "scale"))
    h_v = v.shape[1]
    for n in range(len(cu) - 1):
        for h in range(h_v):
            ts = list(range(cu[n], cu[n + 1]))
            A = np.exp(np.cumsum(g[ts, h]))
            S0, dF = s0[n, h], dfin[n, h]
            dS0 = A[-1] * dF + sum(sc * A[i] * np.outer(q[t, 0], do[t, h]) for i, t in enumerate(ts))
            np.testing.assert_allclose(got["d_initial"][n, h], dS0, rtol=1e-12, atol=1e-12)
            for i, t in enumerate(ts):
                tail = sum(sc * A[j] * q[ts[j], 0] @ S0 @ do[ts[j], h] for j in range(i, len(ts)))
                dg = tail + A[-1] * np.sum(dF * S0)
                np.testing.assert_allclose(got["dg"][t, h], dg, rtol=1e-11, atol=1e-12)
                G = A[-1] / A[i] * dF + sum(sc * A[j] / A[i] * np.outer(q[ts[j], 0], do[ts[j], h])
                                            for j in range(i, len(ts)))
                db = (G.T @ k[t, 0]) @ (v[t, h] - A[i] * S0.T @ k[t, 0])
                np.testing.assert_allclose(got["dbeta"][t, h], db, rtol=1e-11, atol=1e-12)
    # dq sums the group's heads: scale sum_h A_t^(h) S_0^(h) do_t^(h)
    for n in range(len(cu) - 1):
        for t in range(cu[n], cu[n + 1]):
            want = sum(sc * np.exp(np.sum(g[cu[n]:t + 1, h])) * s0[n, h] @ do[t, h] for h in range(h_v))
            np.testing.assert_allclose(got["dq"][t, 0], want, rtol=1e-12, atol=1e-12)


ALL_PINS = [pin_finite_differences, pin_no_write_closed_form]


@pytest.mark.parametrize("form", list(FORMS))
@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_backward_oracle_pins(form, pin):
    pin(FORMS[form])


def test_c_equals_numpy_backward():
    r = np.random.default_rng(5)
    T, h_qk, h_v, d = 200, 2, 4, 16
    q = r.standard_normal((T, h_qk, d))
    k = r.standard_normal((T, h_qk, d)) / 4
    v = r.standard_normal((T, h_v, d))
    g = -r.random((T, h_v))
    b = r.random((T, h_v))
    do = r.standard_normal((T, h_v, d))
    cu = [0, 70, 70, 200]     # includes an empty sequence
    s0 = r.standard_normal((3, h_v, d, d))
    df = r.standard_normal((3, h_v, d, d))
    a = gdn_sequential_bwd(q, k, v, g, b, 0.3, do, s0, df, cu)
    c = gdn_sequential_bwd_np(q, k, v, g, b, 0.3, do, s0, df, cu)
    for key in a:
        np.testing.assert_allclose(a[key], c[key], rtol=1e-11, atol=1e-12)
    # the empty sequence passes its state gradient straight through
    np.testing.assert_array_equal(a["d_initial"][1], df[1])


# --- planted slips in a copy of the reverse pass: the pins must catch each ---

def _mutant(kind):
    def f(q, k, v, g, beta, scale, d_out, s0, dfin, cu):
        T, h_qk, d_k = q.shape
        h_v, d_v = v.shape[1:]
        out = {x: np.zeros((T, h_v, d_k)) for x in ("dq", "dk")}
        dv = np.zeros((T, h_v, d_v))
        dg = np.zeros((T, h_v))
        db = np.zeros((T, h_v))
        dinit = np.zeros((len(cu) - 1, h_v, d_k, d_v))
        for n in range(len(cu) - 1):
            for h in range(h_v):
                hq = h * h_qk // h_v
                states = [s0[n, h].copy()]
                for t in range(cu[n], cu[n + 1]):
                    D = np.exp(g[t, h]) * states[-1]
                    states.append(D + beta[t, h] * np.outer(k[t, hq], v[t, h] - D.T @ k[t, hq]))
                G = dfin[n, h].copy()
                for t in range(cu[n + 1] - 1, cu[n] - 1, -1):
                    Sp, St = states[t - cu[n]], states[t - cu[n] + 1]
                    kt, qt, vt, dot, a, bt = k[t, hq], q[t, hq], v[t, h], d_out[t, h], np.exp(g[t, h]), beta[t, h]
                    out["dq"][t, h] = scale * (Sp if kind == "dq_old_state" else St) @ dot
                    G = G + scale * np.outer(qt, dot)
                    D = a * Sp
                    p = D.T @ kt
                    dw = G.T @ kt
                    out["dk"][t, h] = G @ (bt * (vt - p))
                    db[t, h] = dw @ (vt if kind == "dbeta_drops_p" else vt - p)
                    dv[t, h] = bt * dw
                    dp = (bt if kind == "dp_sign" else -bt) * dw
                    if kind != "no_G_from_p":
                        G = G + np.outer(kt, dp)
                    if kind != "no_dk_from_p":
                        out["dk"][t, h] += D @ dp
                    dg[t, h] = np.sum(G * (Sp if kind == "dg_undecayed" else D))
                    if kind != "no_G_decay":
                        G = a * G
                dinit[n, h] = G
        gs = lambda x: x.reshape(T, h_qk, h_v // h_qk, d_k).sum(axis=2)  # noqa: E731
        return dict(dq=gs(out["dq"]), dk=gs(out["dk"]), dv=dv, dg=dg, dbeta=db, d_initial=dinit)
    return f


BWD_MUTANTS = ["dq_old_state", "dbeta_drops_p", "dp_sign", "no_G_from_p", "no_dk_from_p",
               "dg_undecayed", "no_G_decay"]


def test_backward_mutant_baseline_passes():
    for pin in ALL_PINS:
        pin(_mutant("none"))


@pytest.mark.parametrize("kind", BWD_MUTANTS)
def test_backward_planted_mistake_is_caught(kind):
    failed = []
    for pin in ALL_PINS:
        try:
            pin(_mutant(kind))
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"no pin catches the planted mistake {kind!r}"
