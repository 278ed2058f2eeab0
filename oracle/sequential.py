"""Sequential fp64 oracle: the gated delta rule applied token by token.

Test infrastructure only (see the package docstring).

The FlashQLA page ("FlashQLA: CP-/Bwd-friendly fused linear attention kernels for
GDN", section on optimising GDN chunked prefill) accelerates the chunked prefill of
the Gated DeltaNet recurrence. The recurrence is the gated delta rule
    S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,   o_t = S_t q_t.
Both implementations here store the transposed state (d_k x d_v) and apply, per
token: decay by a_t = exp(g_t); error e = v_t - S^T k_t; S += b_t k_t e^T;
o_t = scale * S^T q_t (read-out after the update). Value head h reads query/key
head floor(h * h_qk / h_v).

``gdn_sequential`` runs the C implementation in ``gdn_oracle.c`` (threads over
(sequence, head) pairs); ``gdn_sequential_np`` is the same definition in numpy for
small inputs.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_BUILD = os.path.join(_HERE, "_build")
_LIB = os.path.join(_BUILD, "libgdn_oracle.so")
_lock = threading.Lock()
_lib = None


def lib_path() -> str:
    return _LIB


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (host code only)."""
    os.makedirs(_BUILD, exist_ok=True)
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-o", tmp, _SRC,
                               "-lpthread", "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB)
            f = lib.gdn_oracle_fwd
            P = ctypes.c_void_p
            I = ctypes.c_int64
            f.argtypes = [I, P, I, I, I, I, P, P, P, P, P, ctypes.c_double, P, P, P,
                          I, I, P, ctypes.c_int]
            f.restype = ctypes.c_int
            _lib = lib
    return _lib


def _f64(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _default_threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def gdn_sequential(q, k, v, g, beta, scale, initial_state=None, cu_seqlens=None,
                   snap_stride=0, n_snap=0, n_threads=None):
    """Run the C oracle.

    q, k: [T, h_qk, d_k]; v: [T, h_v, d_v]; g, beta: [T, h_v] (any float dtype,
    converted to fp64). cu_seqlens: None (one sequence) or n_seqs+1 token offsets.
    initial_state: None or [n_seqs, h_v, d_k, d_v].
    Returns (o [T, h_v, d_v], final_state [n_seqs, h_v, d_k, d_v], snaps or None)
    where snaps[n, h, j] is the state after j*snap_stride tokens of sequence n.
    """
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    T, h_qk, d_k = q.shape
    h_v, d_v = v.shape[1], v.shape[2]
    assert k.shape == q.shape and v.shape[0] == T and g.shape == (T, h_v) == beta.shape
    if cu_seqlens is None:
        cu = np.array([0, T], dtype=np.int64)
    else:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    n_seqs = len(cu) - 1
    assert cu[0] == 0 and cu[-1] == T
    s0 = None if initial_state is None else _f64(initial_state)
    if s0 is not None:
        assert s0.shape == (n_seqs, h_v, d_k, d_v)
    out = np.zeros((T, h_v, d_v), dtype=np.float64)
    fin = np.zeros((n_seqs, h_v, d_k, d_v), dtype=np.float64)
    snaps = None
    if snap_stride > 0 and n_snap > 0:
        snaps = np.zeros((n_seqs, h_v, n_snap, d_k, d_v), dtype=np.float64)
    rc = _load().gdn_oracle_fwd(n_seqs, _ptr(cu), h_qk, h_v, d_k, d_v, _ptr(q), _ptr(k),
                                _ptr(v), _ptr(g), _ptr(beta), float(scale), _ptr(s0),
                                _ptr(out), _ptr(fin), int(snap_stride), int(n_snap),
                                _ptr(snaps), int(n_threads or _default_threads()))
    if rc != 0:
        raise RuntimeError(f"gdn_oracle_fwd failed with code {rc}")
    return out, fin, snaps


def gdn_sequential_np(q, k, v, g, beta, scale, initial_state=None, cu_seqlens=None):
    """numpy form of the same token loop (small inputs only).

    Returns (o, final_state, states) where states[n][h] is the list of states
    after each token of sequence n (index 0 = initial state).
    """
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    T, h_qk, d_k = q.shape
    h_v, d_v = v.shape[1], v.shape[2]
    cu = [0, T] if cu_seqlens is None else [int(x) for x in cu_seqlens]
    n_seqs = len(cu) - 1
    out = np.zeros((T, h_v, d_v))
    fin = np.zeros((n_seqs, h_v, d_k, d_v))
    states = [[None] * h_v for _ in range(n_seqs)]
    for n in range(n_seqs):
        for h in range(h_v):
            hq = h * h_qk // h_v
            S = np.zeros((d_k, d_v)) if initial_state is None else _f64(initial_state[n, h]).copy()
            hist = [S.copy()]
            for t in range(cu[n], cu[n + 1]):
                kt, qt, vt = k[t, hq], q[t, hq], v[t, h]
                S = np.exp(g[t, h]) * S                      # decay
                e = vt - S.T @ kt                            # prediction error
                S = S + beta[t, h] * np.outer(kt, e)         # delta-rule update
                out[t, h] = scale * (S.T @ qt)               # read-out after update
                hist.append(S.copy())
            fin[n, h] = S
            states[n][h] = hist
    return out, fin, states
