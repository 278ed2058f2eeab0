"""fp64 model of the chunked (WY) form and of intra-card context parallelism.

Test infrastructure only (see the package docstring). Everything is plain numpy
in fp64, one (sequence, value head) and one chunk at a time, in the order the
method states its steps.

Sources. The FlashQLA pages ("FlashQLA: CP-/Bwd-friendly fused linear attention
kernels for GDN"):
  * section on optimising GDN chunked prefill: the prefill runs chunk-wise and
    the standard flow round-trips the intermediates W, U and S through HBM;
    FlashQLA splits the forward into two fused kernels with a context-parallel
    preprocessing step between them;
  * section "Gate-Driven Automatic Intra-Card Context Parallelism (AutoCP)":
    the sequence is cut into CP ranks of L chunks each; each rank's initial
    state S0 comes either from the expensive correction matrix M or, for heads
    whose gates decay fast, from a 6-8 chunk warm-up that pushes the state
    error below a noise floor;
  * section on the warp-specialised kernels, "Forward Pass" and "CP
    Preprocessing": the forward computes V' (pseudo-values), S and O per chunk.
The pages give none of the formulas. The chunked form below is the standard WY
form of the gated delta rule, derived from the token recurrence
    S <- a S;  S <- S + b k (v - S^T k)^T;  o = scale S^T q
(state stored d_k x d_v). For one chunk of c tokens with incoming state S:
    gamma     = cumsum(g)                         (gate log-decay inside the chunk)
    A[i, j]   = b_i exp(gamma_i - gamma_j) k_i.k_j   for i > j, else 0
    T         = (I + A)^-1
    W         = T diag(b exp(gamma)) K,   U = T diag(b) V
    V'        = U - W S                           (the pseudo-values)
    O         = scale (diag(exp(gamma)) Q S + (Q K^T * D) V'),
                D[r, i] = exp(gamma_r - gamma_i) for i <= r, else 0
    S_next    = exp(gamma_c) S + Kt^T V',  Kt = diag(exp(gamma_c - gamma)) K
Equivalently S_next = M_c S + H_c with M_c = exp(gamma_c) I - Kt^T W and
H_c = Kt^T U; a segment's map is the composition of its chunks' maps.
"""
from __future__ import annotations

import math

import numpy as np

CHUNK = 64


def chunk_prep(k, v, g, beta):
    """Per-chunk quantities that do not depend on the state.

    k: [c, d_k], v: [c, d_v], g, beta: [c] (c <= CHUNK). Returns gamma, A, T, W, U.
    """
    k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (k, v, g, beta))
    c = k.shape[0]
    gamma = np.cumsum(g)
    lower = np.tril(np.ones((c, c), dtype=bool), -1)
    diff = np.where(lower, gamma[:, None] - gamma[None, :], -np.inf)
    A = beta[:, None] * np.exp(diff) * (k @ k.T)
    T = np.linalg.inv(np.eye(c) + A)
    W = T @ ((beta * np.exp(gamma))[:, None] * k)
    U = T @ (beta[:, None] * v)
    return gamma, A, T, W, U


def chunk_forward(S, q, k, gamma, W, U, scale):
    """One chunk given its prep quantities and the incoming state S [d_k, d_v].

    Returns (O [c, d_v], S_next, V').
    """
    q, k = np.asarray(q, dtype=np.float64), np.asarray(k, dtype=np.float64)
    c = q.shape[0]
    Vp = U - W @ S
    causal = np.tril(np.ones((c, c), dtype=bool))
    D = np.exp(np.where(causal, gamma[:, None] - gamma[None, :], -np.inf))
    O = scale * (np.exp(gamma)[:, None] * q @ S + ((q @ k.T) * D) @ Vp)
    Kt = np.exp(gamma[-1] - gamma)[:, None] * k
    S_next = math.exp(gamma[-1]) * S + Kt.T @ Vp
    return O, S_next, Vp


def chunk_affine(k, gamma, W, U):
    """The chunk's state map S -> M S + H."""
    k = np.asarray(k, dtype=np.float64)
    Kt = np.exp(gamma[-1] - gamma)[:, None] * k
    M = math.exp(gamma[-1]) * np.eye(k.shape[1]) - Kt.T @ W
    H = Kt.T @ U
    return M, H


def n_chunks(length):
    return (int(length) + CHUNK - 1) // CHUNK


def segments(N, L):
    """Chunk ranges [a_s, a_{s+1}) of the P = ceil(N / L) segments of L chunks."""
    if N == 0:
        return []
    P = (N + L - 1) // L
    return [(s * L, min((s + 1) * L, N)) for s in range(P)]


def warmup_window(a, w, g_seq=None, eps=None):
    """Chunk window [lo, a) scanned to approximate the state at chunk a.

    Without gates: the w chunks before a. A window reaching chunk 0 makes the
    warm-up exact (it starts from the sequence's initial state), so when
    a <= w the window is [0, a). With gates (g_seq, eps): the shortest run of
    whole chunks before a, at most w, whose total log-decay sum(g) is at most
    ln(eps) -- the gate has then already damped the state the scan misses to
    below the noise floor; if no run of up to w chunks qualifies, the w chunks
    before a (the AutoCP section's warm-up of a fixed number of chunks, read
    as an upper bound on the window)."""
    if a - w <= 0:
        return 0, a
    if g_seq is not None:
        cum = 0.0
        for j in range(1, w + 1):
            cum += float(np.sum(g_seq[(a - j) * CHUNK:(a - j + 1) * CHUNK]))
            if cum <= math.log(eps):
                return a - j, a
    return a - w, a


def choose_path(g_seq, N, L, w, eps):
    """Path of one (sequence, value head): 'warmup' iff at every segment boundary
    whose window does not reach the sequence start, the window's total log-decay
    sum(g) is at most ln(eps); else 'exact'."""
    for a, _ in segments(N, L)[1:]:
        lo, hi = warmup_window(a, w)
        if lo == 0:
            continue
        if float(np.sum(g_seq[lo * CHUNK:hi * CHUNK])) > math.log(eps):
            return "exact"
    return "warmup"


def boundary_rule(g_seq, a, w, eps):
    """Decision for the segment boundary at chunk a under the per-boundary
    reading of the AutoCP section (gates decide per boundary, not per head):
      ('start', a)   the w-chunk window reaches the sequence start: warm up over
                     [0, a) from the initial state, which is exact;
      ('warmup', j)  j <= w is the shortest run of whole chunks before a whose
                     total log-decay sum(g) is at most ln(eps): warm up over
                     [a - j, a) from zero -- the state the scan misses has been
                     damped below the noise floor;
      ('exact', 0)   no run of up to w chunks decays that far: the boundary
                     state comes from the previous segment's exact map."""
    if a - w <= 0:
        return "start", a
    cum = 0.0
    for j in range(1, w + 1):
        cum += float(np.sum(g_seq[(a - j) * CHUNK:(a - j + 1) * CHUNK]))
        if cum <= math.log(eps):
            return "warmup", j
    return "exact", 0


def boundary_summary(kinds):
    """Path code of one (sequence, head) over its boundaries' decisions, the
    boundaries whose window reaches the sequence start left out: 1 all warmed
    up, 0 all exact, 2 mixed, 3 no such boundary."""
    ks = [k for k, _ in kinds if k != "start"]
    if not ks:
        return 3
    if all(k == "warmup" for k in ks):
        return 1
    if all(k == "exact" for k in ks):
        return 0
    return 2


def _head_inputs(q, k, v, g, beta, t0, t1, h, hq):
    return q[t0:t1, hq], k[t0:t1, hq], v[t0:t1, h], g[t0:t1, h], beta[t0:t1, h]


def chunked_forward(q, k, v, g, beta, scale, initial_state=None, cu_seqlens=None,
                    L=None, mode="off", w=6, eps=1e-4):
    """Chunked forward with optional context parallelism.

    q, k: [T, h_qk, d_k]; v: [T, h_v, d_v]; g, beta: [T, h_v].
    mode: 'off' (one segment per sequence), 'exact' (segment initial states by
    composing the chunk maps: S0(s+1) = M_s S0(s) + H_s), 'warmup' (each
    boundary state by scanning the w chunks before it from zero), 'auto'
    (per (sequence, head) via ``choose_path``), 'boundary' (per boundary via
    ``boundary_rule``: a warm-up or start boundary takes its scanned state, an
    exact one the previous segment's map applied to the previous boundary's
    state, whichever way that one was obtained).
    Returns (o, final_state, info) with info['S0'][n][h] = list of segment
    initial states and info['path'][n][h] (for 'boundary' the code of
    ``boundary_summary``, and info['boundary'][n][h] the decisions).
    """
    q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
    T, h_qk, d_k = q.shape
    h_v, d_v = v.shape[1], v.shape[2]
    cu = [0, T] if cu_seqlens is None else [int(x) for x in cu_seqlens]
    n_seqs = len(cu) - 1
    o = np.zeros((T, h_v, d_v))
    fin = np.zeros((n_seqs, h_v, d_k, d_v))
    info = {"S0": [[None] * h_v for _ in range(n_seqs)],
            "path": [[None] * h_v for _ in range(n_seqs)],
            "boundary": [[None] * h_v for _ in range(n_seqs)]}
    for n in range(n_seqs):
        t0, t1 = cu[n], cu[n + 1]
        N = n_chunks(t1 - t0)
        Ls = N if (mode == "off" or L is None) else int(L)
        Ls = max(Ls, 1)
        segs = segments(N, Ls)
        for h in range(h_v):
            hq = h * h_qk // h_v
            qs, ks, vs, gs, bs = _head_inputs(q, k, v, g, beta, t0, t1, h, hq)
            S_init = (np.zeros((d_k, d_v)) if initial_state is None
                      else np.asarray(initial_state[n, h], dtype=np.float64).copy())
            prep = []
            for c in range(N):
                sl = slice(c * CHUNK, min((c + 1) * CHUNK, t1 - t0))
                prep.append((sl,) + chunk_prep(ks[sl], vs[sl], gs[sl], bs[sl]))

            path = mode
            if mode == "auto":
                path = choose_path(gs, N, Ls, w, eps)
            elif mode == "off":
                path = "exact"
            info["path"][n][h] = path

            # segment initial states
            S0 = [S_init]
            if path == "boundary":
                kinds = []
                for s_ in range(1, len(segs)):
                    a = segs[s_][0]
                    kind, j = boundary_rule(gs, a, w, eps)
                    kinds.append((kind, j))
                    if kind == "exact":
                        M = np.eye(d_k)
                        Hm = np.zeros((d_k, d_v))
                        for c in range(segs[s_ - 1][0], segs[s_ - 1][1]):
                            sl, gam, _, _, W, U = prep[c]
                            Mc, Hc = chunk_affine(ks[sl], gam, W, U)
                            M, Hm = Mc @ M, Mc @ Hm + Hc
                        S0.append(M @ S0[-1] + Hm)
                    else:
                        lo = 0 if kind == "start" else a - j
                        S = S_init.copy() if kind == "start" else np.zeros((d_k, d_v))
                        for c in range(lo, a):
                            sl, gam, _, _, W, U = prep[c]
                            _, S, _ = chunk_forward(S, qs[sl], ks[sl], gam, W, U, scale)
                        S0.append(S)
                info["boundary"][n][h] = kinds
                info["path"][n][h] = boundary_summary(kinds)
            elif path == "exact":
                for (a, b_) in segs[:-1]:
                    M = np.eye(d_k)
                    Hm = np.zeros((d_k, d_v))
                    for c in range(a, b_):
                        sl, gam, _, _, W, U = prep[c]
                        Mc, Hc = chunk_affine(ks[sl], gam, W, U)
                        M, Hm = Mc @ M, Mc @ Hm + Hc
                    S0.append(M @ S0[-1] + Hm)
            elif path == "warmup":
                for (a, _) in segs[1:]:
                    lo, hi = warmup_window(a, w, gs, eps)
                    S = S_init.copy() if lo == 0 else np.zeros((d_k, d_v))
                    for c in range(lo, hi):
                        sl, gam, _, _, W, U = prep[c]
                        _, S, _ = chunk_forward(S, qs[sl], ks[sl], gam, W, U, scale)
                    S0.append(S)
            else:
                raise ValueError(f"unknown mode {mode!r}")
            info["S0"][n][h] = S0

            # the forward scan of every segment from its initial state
            S = S_init
            for s, (a, b_) in enumerate(segs):
                S = S0[s].copy()
                for c in range(a, b_):
                    sl, gam, _, _, W, U = prep[c]
                    O, S, _ = chunk_forward(S, qs[sl], ks[sl], gam, W, U, scale)
                    o[t0 + sl.start:t0 + sl.stop, h] = O
            fin[n, h] = S
    return o, fin, info


def prep_all(k, v, g, beta, h_v, cu_seqlens=None):
    """gamma, W, U of every (chunk, value head), zero-padded to CHUNK rows.

    Chunks are numbered sequence by sequence (a sequence of length l has
    ceil(l / CHUNK) chunks). Rows past a short final chunk are what padding
    with g = 0, beta = 0, k = v = 0 gives: gamma stays at its last value and
    the W, U rows are zero. Returns gamma [n_chunks, h_v, CHUNK],
    W [n_chunks, h_v, CHUNK, d_k], U [n_chunks, h_v, CHUNK, d_v].
    """
    k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (k, v, g, beta))
    T, h_qk, d_k = k.shape
    d_v = v.shape[2]
    cu = [0, T] if cu_seqlens is None else [int(x) for x in cu_seqlens]
    total = sum(n_chunks(cu[i + 1] - cu[i]) for i in range(len(cu) - 1))
    G = np.zeros((total, h_v, CHUNK))
    Wa = np.zeros((total, h_v, CHUNK, d_k))
    Ua = np.zeros((total, h_v, CHUNK, d_v))
    ci = 0
    for n in range(len(cu) - 1):
        t0, t1 = cu[n], cu[n + 1]
        for c in range(n_chunks(t1 - t0)):
            a, b_ = t0 + c * CHUNK, min(t0 + (c + 1) * CHUNK, t1)
            for h in range(h_v):
                hq = h * h_qk // h_v
                gam, _, _, W, U = chunk_prep(k[a:b_, hq], v[a:b_, h], g[a:b_, h], beta[a:b_, h])
                G[ci, h, :b_ - a] = gam
                G[ci, h, b_ - a:] = gam[-1]   # padding rows carry g = 0
                Wa[ci, h, :b_ - a] = W
                Ua[ci, h, :b_ - a] = U
            ci += 1
    return G, Wa, Ua
