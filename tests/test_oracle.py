"""The fp64 oracle against its pins (CPU only)."""
from __future__ import annotations

import numpy as np
import pytest

from oracle import gdn_sequential, gdn_sequential_np
from oracle_pins import ALL_PINS


def c_oracle(q, k, v, g, b, scale, S0, cu):
    o, S, _ = gdn_sequential(q, k, v, g, b, scale, S0, cu, n_threads=2)
    return o, S


def np_oracle(q, k, v, g, b, scale, S0, cu):
    o, S, _ = gdn_sequential_np(q, k, v, g, b, scale, S0, cu)
    return o, S


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_c_oracle_pins(pin):
    pin(c_oracle)


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_numpy_oracle_pins(pin):
    pin(np_oracle)


def test_c_equals_numpy_on_random_varlen():
    r = np.random.default_rng(11)
    T, h_qk, h_v, d_k, d_v = 50, 2, 4, 8, 5
    q = r.standard_normal((T, h_qk, d_k))
    k = r.standard_normal((T, h_qk, d_k)) / 3
    v = r.standard_normal((T, h_v, d_v))
    g = -r.uniform(0, 1, (T, h_v))
    b = r.uniform(0, 1, (T, h_v))
    cu = [0, 17, 17, 40, 50]
    S0 = r.standard_normal((4, h_v, d_k, d_v))
    o1, S1, snaps = gdn_sequential(q, k, v, g, b, 0.3, S0, cu, snap_stride=8, n_snap=4)
    o2, S2, hist = gdn_sequential_np(q, k, v, g, b, 0.3, S0, cu)
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(S1, S2, atol=1e-13)
    for n in range(4):
        ln = cu[n + 1] - cu[n]
        for h in range(h_v):
            for j in range(4):
                if j * 8 <= ln:
                    np.testing.assert_allclose(snaps[n, h, j], hist[n][h][j * 8], atol=1e-13)


# --- planted mistakes: every plausible slip in the recurrence must trip a pin ---

def _mutant(kind):
    def f(q, k, v, g, b, scale, S0, cu):
        q, k, v, g, b = (np.asarray(x, float) for x in (q, k, v, g, b))
        T, h_qk, d_k = q.shape
        h_v, d_v = v.shape[1:]
        cuv = [0, T] if cu is None else [int(x) for x in cu]
        out = np.zeros((T, h_v, d_v))
        fin = np.zeros((len(cuv) - 1, h_v, d_k, d_v))
        for n in range(len(cuv) - 1):
            for h in range(h_v):
                hq = (h % h_qk) if kind == "head_map" else h * h_qk // h_v
                S = np.zeros((d_k, d_v)) if S0 is None else np.array(S0[n, h], float)
                for t in range(cuv[n], cuv[n + 1]):
                    kt, qt, vt, a, bt = k[t, hq], q[t, hq], v[t, h], np.exp(g[t, h]), b[t, h]
                    if kind == "readout_before_update":
                        out[t, h] = scale * (a * S).T @ qt
                    if kind == "decay_after_error":
                        e = vt - S.T @ kt
                        S = a * S + bt * np.outer(kt, e)
                    elif kind == "no_beta_on_error":
                        S = a * S
                        e = vt - bt * (S.T @ kt)
                        S = S + bt * np.outer(kt, e)
                    elif kind == "transposed_readout":
                        S = a * S
                        e = vt - S.T @ kt
                        S = S + bt * np.outer(kt, e)
                    elif kind == "sign_flip":
                        S = a * S
                        e = vt + S.T @ kt
                        S = S + bt * np.outer(kt, e)
                    else:
                        S = a * S
                        e = vt - S.T @ kt
                        S = S + bt * np.outer(kt, e)
                    if kind == "transposed_readout":
                        out[t, h] = scale * (S @ qt if d_v == d_k else S.T @ qt)
                    elif kind != "readout_before_update":
                        out[t, h] = scale * S.T @ qt
                fin[n, h] = S
        return out, fin
    return f


MUTANTS = ["readout_before_update", "decay_after_error", "no_beta_on_error",
           "transposed_readout", "sign_flip", "head_map"]


def test_mutant_baseline_passes():
    f = _mutant("none")
    for pin in ALL_PINS:
        pin(f)


@pytest.mark.parametrize("kind", MUTANTS)
def test_planted_mistake_is_caught(kind):
    f = _mutant(kind)
    failed = []
    for pin in ALL_PINS:
        try:
            pin(f)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"no pin catches the planted mistake {kind!r}"
