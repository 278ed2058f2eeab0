"""fp64 gradients of the gated delta rule (test infrastructure only).

The FlashQLA page ("FlashQLA: CP-/Bwd-friendly fused linear attention kernels for
GDN") is about kernels whose backward pass is also fast, but prints no backward
formulas. The backward of the forward pass is, by definition, the gradient of the
sequential recurrence (see ``sequential``) with respect to its inputs, given
dL/do for every token and dL/dS for the final state. Two implementations:

``gdn_sequential_bwd`` runs ``gdn_oracle_bwd`` in ``gdn_oracle.c`` (reverse mode
through the token loop, states recomputed from a checkpoint every 64 tokens,
threads over (sequence, head) pairs); ``gdn_sequential_bwd_np`` is the same
reverse pass in numpy over all stored states, for small inputs. Per token, with
D = exp(g) S_prev, p = D^T k, w = beta (v - p), S = D + k w^T, o = scale S^T q
and G the running dL/dS, the reverse steps are
    G += scale q do^T;  dq = scale S do
    dw = G^T k;  dk = G w;  dbeta = dw . (v - p);  dv = beta dw;  dp = -beta dw
    G += k dp^T;  dk += D dp;  dg = <G, D>;  G <- exp(g) G
Query/key gradients are summed over the value heads of a group
(value head h reads query/key head floor(h * h_qk / h_v)).
"""
from __future__ import annotations

import ctypes

import numpy as np

from .sequential import _default_threads, _f64, _load, _ptr


def _lib():
    lib = _load()
    f = lib.gdn_oracle_bwd
    if not f.argtypes:
        P = ctypes.c_void_p
        I = ctypes.c_int64
        f.argtypes = [I, P, I, I, I, I, P, P, P, P, P, ctypes.c_double, P, P, P,
                      P, P, P, P, P, P, ctypes.c_int]
        f.restype = ctypes.c_int
    return lib


def _group_sum(part, h_qk):
    """[T, h_v, d] per-value-head parts -> [T, h_qk, d] summed over each group."""
    T, h_v, d = part.shape
    return part.reshape(T, h_qk, h_v // h_qk, d).sum(axis=2)


def gdn_sequential_bwd(q, k, v, g, beta, scale, d_out, initial_state=None, d_final=None,
                       cu_seqlens=None, n_threads=None):
    """Gradients from the C oracle.

    Shapes as ``gdn_sequential`` (token axis merged), d_out like v, d_final and
    initial_state [n_seqs, h_v, d_k, d_v] or None. Returns a dict with dq, dk
    [T, h_qk, d_k], dv [T, h_v, d_v], dg, dbeta [T, h_v] and d_initial
    [n_seqs, h_v, d_k, d_v]."""
    q, k, v, g, beta, d_out = map(_f64, (q, k, v, g, beta, d_out))
    T, h_qk, d_k = q.shape
    h_v, d_v = v.shape[1], v.shape[2]
    assert d_out.shape == v.shape
    cu = np.array([0, T], dtype=np.int64) if cu_seqlens is None else \
        np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    n_seqs = len(cu) - 1
    assert cu[0] == 0 and cu[-1] == T
    s0 = None if initial_state is None else _f64(initial_state)
    dfin = None if d_final is None else _f64(d_final)
    for x in (s0, dfin):
        if x is not None:
            assert x.shape == (n_seqs, h_v, d_k, d_v)
    dq = np.zeros((T, h_v, d_k))
    dk = np.zeros((T, h_v, d_k))
    dv = np.zeros((T, h_v, d_v))
    dg = np.zeros((T, h_v))
    db = np.zeros((T, h_v))
    dinit = np.zeros((n_seqs, h_v, d_k, d_v))
    rc = _lib().gdn_oracle_bwd(n_seqs, _ptr(cu), h_qk, h_v, d_k, d_v, _ptr(q), _ptr(k), _ptr(v),
                               _ptr(g), _ptr(beta), float(scale), _ptr(s0), _ptr(d_out), _ptr(dfin),
                               _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(db), _ptr(dinit),
                               int(n_threads or _default_threads()))
    if rc != 0:
        raise RuntimeError(f"gdn_oracle_bwd failed with code {rc}")
    return dict(dq=_group_sum(dq, h_qk), dk=_group_sum(dk, h_qk), dv=dv, dg=dg, dbeta=db,
                d_initial=dinit)


def gdn_sequential_bwd_np(q, k, v, g, beta, scale, d_out, initial_state=None, d_final=None,
                          cu_seqlens=None):
    """The same gradients in numpy, storing every state (small inputs only)."""
    q, k, v, g, beta, d_out = map(_f64, (q, k, v, g, beta, d_out))
    T, h_qk, d_k = q.shape
    h_v, d_v = v.shape[1], v.shape[2]
    cu = [0, T] if cu_seqlens is None else [int(x) for x in cu_seqlens]
    n_seqs = len(cu) - 1
    dq = np.zeros((T, h_v, d_k))
    dk = np.zeros((T, h_v, d_k))
    dv = np.zeros((T, h_v, d_v))
    dg = np.zeros((T, h_v))
    db = np.zeros((T, h_v))
    dinit = np.zeros((n_seqs, h_v, d_k, d_v))
    for n in range(n_seqs):
        for h in range(h_v):
            hq = h * h_qk // h_v
            S = np.zeros((d_k, d_v)) if initial_state is None else _f64(initial_state[n, h]).copy()
            states = [S]
            for t in range(cu[n], cu[n + 1]):
                D = np.exp(g[t, h]) * states[-1]
                p = D.T @ k[t, hq]
                states.append(D + beta[t, h] * np.outer(k[t, hq], v[t, h] - p))
            G = np.zeros((d_k, d_v)) if d_final is None else _f64(d_final[n, h]).copy()
            for t in range(cu[n + 1] - 1, cu[n] - 1, -1):
                i = t - cu[n]
                Sp, St = states[i], states[i + 1]
                kt, qt, vt, dot = k[t, hq], q[t, hq], v[t, h], d_out[t, h]
                a, bt = np.exp(g[t, h]), beta[t, h]
                dq[t, h] = scale * St @ dot
                G = G + scale * np.outer(qt, dot)
                D = a * Sp
                p = D.T @ kt
                w = bt * (vt - p)
                dw = G.T @ kt
                dk[t, h] = G @ w
                db[t, h] = dw @ (vt - p)
                dv[t, h] = bt * dw
                dp = -bt * dw
                G = G + np.outer(kt, dp)
                dk[t, h] += D @ dp
                dg[t, h] = np.sum(G * D)
                G = a * G
            dinit[n, h] = G
    return dict(dq=_group_sum(dq, h_qk), dk=_group_sum(dk, h_qk), dv=dv, dg=dg, dbeta=db,
                d_initial=dinit)
