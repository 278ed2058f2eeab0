"""Seeded synthetic inputs for the Gated DeltaNet forward.

This module only draws random numbers and rounds them to the input dtype; it
holds none of the method's arithmetic. Both the tests (which feed the same
arrays to the fp64 oracle) and the benchmark use it.

Recipe (all configurations):
  * numpy PCG64 streams from SeedSequence(seed).spawn(7): one each for q, k, v,
    beta, g, the fast/slow head permutation and the initial state.
  * q, k ~ N(0, 1) in fp64, L2-normalised over d_k per (token, query/key head),
    then rounded to the input dtype (bf16: fp64 -> fp32 -> bf16, round to
    nearest even at each step). v ~ N(0, 1), rounded the same way.
  * beta = sigmoid(N(0, 1)) in fp32.
  * g = log(alpha) per token and value head, fp32, from the head's class:
      'plain'  -softplus(N(0, 1))
      'fast'   -softplus(N(1, 0.5))          (mean about -1.34 per token)
      'slow'   -U(1e-4, 1e-3)
      'near1'  -U(1e-5, 1e-4)
    where softplus(x) = log1p(exp(-|x|)) + max(x, 0). Heads are assigned to
    classes by a seeded permutation: the first round(fast_frac * h_v) heads of
    the permutation are fast, the rest take the slow class.
  * initial state: zero, or N(0, init_std) in fp32, shape [n_seqs, h_v, d_k, d_v].
  * scale = 1 / sqrt(d_k).
Stored arrays are fp32 holding exactly the values of the input dtype.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

_BLOCK = 8192  # tokens drawn per call; the streams are consumed in token order


def round_bf16(x) -> np.ndarray:
    """fp64/fp32 -> bf16 values (as fp32), round to nearest even."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    b = x.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32).reshape(x.shape)


def _softplus(x):
    return np.log1p(np.exp(-np.abs(x))) + np.maximum(x, 0.0)


@dataclasses.dataclass
class Inputs:
    q: np.ndarray          # [B, T, h_qk, d_k] fp32 (values exact in io dtype)
    k: np.ndarray
    v: np.ndarray          # [B, T, h_v, d_v]
    g: np.ndarray          # [B, T, h_v] fp32
    beta: np.ndarray       # [B, T, h_v] fp32
    initial_state: Optional[np.ndarray]   # [n_seqs, h_v, d_k, d_v] fp32 or None
    scale: float
    io_dtype: str          # 'bf16' or 'f32'
    cu_seqlens: Optional[np.ndarray]      # int32 [n_seqs + 1] (B == 1) or None
    head_class: list       # class name per value head
    name: str = ""

    @property
    def B(self):
        return self.q.shape[0]

    @property
    def T(self):
        return self.q.shape[1]

    @property
    def h_qk(self):
        return self.q.shape[2]

    @property
    def h_v(self):
        return self.v.shape[2]

    @property
    def n_seqs(self):
        return self.B if self.cu_seqlens is None else len(self.cu_seqlens) - 1

    def flat_cu(self):
        """Token offsets of the sequences in the flattened [B*T] token axis."""
        if self.cu_seqlens is not None:
            return np.asarray(self.cu_seqlens, dtype=np.int64)
        return np.arange(self.B + 1, dtype=np.int64) * self.T

    def flat(self):
        """(q, k, v, g, beta) with batch and time merged into one token axis."""
        BT = self.B * self.T
        return (self.q.reshape(BT, self.h_qk, -1), self.k.reshape(BT, self.h_qk, -1),
                self.v.reshape(BT, self.h_v, -1), self.g.reshape(BT, self.h_v),
                self.beta.reshape(BT, self.h_v))


def make_inputs(B, T, h_qk, h_v, d_k=128, d_v=128, io_dtype="bf16", seed=0,
                gate="plain", fast_frac=0.7, slow_class="slow", init_std=None,
                cu_seqlens=None, name="") -> Inputs:
    """Draw one workload. gate='plain' gives every head the 'plain' class;
    gate='mixed' splits heads into 'fast' and ``slow_class`` by ``fast_frac``."""
    assert h_v % h_qk == 0
    ss = np.random.SeedSequence(seed).spawn(7)
    rq, rk, rv, rb, rg, rp, rs = (np.random.Generator(np.random.PCG64(s)) for s in ss)
    rnd = round_bf16 if io_dtype == "bf16" else (lambda a: np.asarray(a, dtype=np.float32))

    if gate == "plain":
        classes = ["plain"] * h_v
    elif gate == "mixed":
        perm = rp.permutation(h_v)
        n_fast = int(math.floor(fast_frac * h_v + 0.5))
        classes = [slow_class] * h_v
        for h in perm[:n_fast]:
            classes[int(h)] = "fast"
    else:
        classes = [gate] * h_v

    q = np.empty((B, T, h_qk, d_k), np.float32)
    k = np.empty((B, T, h_qk, d_k), np.float32)
    v = np.empty((B, T, h_v, d_v), np.float32)
    g = np.empty((B, T, h_v), np.float32)
    beta = np.empty((B, T, h_v), np.float32)
    for b in range(B):
        for t0 in range(0, T, _BLOCK):
            t1 = min(t0 + _BLOCK, T)
            n = t1 - t0
            for rr, dst in ((rq, q), (rk, k)):
                x = rr.standard_normal((n, h_qk, d_k))
                x /= np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
                dst[b, t0:t1] = rnd(x)
            v[b, t0:t1] = rnd(rv.standard_normal((n, h_v, d_v)))
            beta[b, t0:t1] = (1.0 / (1.0 + np.exp(-rb.standard_normal((n, h_v))))).astype(np.float32)
            zn = rg.standard_normal((n, h_v))
            zu = rg.random((n, h_v))
            gg = np.empty((n, h_v))
            for h, c in enumerate(classes):
                if c == "plain":
                    gg[:, h] = -_softplus(zn[:, h])
                elif c == "fast":
                    gg[:, h] = -_softplus(1.0 + 0.5 * zn[:, h])
                elif c == "slow":
                    gg[:, h] = -(1e-4 + (1e-3 - 1e-4) * zu[:, h])
                elif c == "near1":
                    gg[:, h] = -(1e-5 + (1e-4 - 1e-5) * zu[:, h])
                else:
                    raise ValueError(c)
            g[b, t0:t1] = gg.astype(np.float32)

    n_seqs = B if cu_seqlens is None else len(cu_seqlens) - 1
    s0 = None
    if init_std is not None:
        s0 = (init_std * rs.standard_normal((n_seqs, h_v, d_k, d_v))).astype(np.float32)
    cu = None if cu_seqlens is None else np.asarray(cu_seqlens, dtype=np.int32)
    if cu is not None:
        assert B == 1 and cu[0] == 0 and cu[-1] == T
    return Inputs(q, k, v, g, beta, s0, 1.0 / math.sqrt(d_k), io_dtype, cu, classes, name)


# The five workloads (sizes as the FlashQLA benchmark table's per-GPU shapes:
# one 32768-token prompt at the TP8, TP2 and TP1 head counts, plus a tiny fp32
# case and a 262144-token long-context case).
CONFIGS = {
    "tiny":   dict(B=1, T=512, h_qk=1, h_v=1, io_dtype="f32", seed=1, gate="plain"),
    "tp8":    dict(B=1, T=32768, h_qk=2, h_v=8, seed=2, gate="mixed"),
    "tp4":    dict(B=1, T=32768, h_qk=4, h_v=16, seed=6, gate="mixed"),
    "tp2":    dict(B=1, T=32768, h_qk=8, h_v=24, seed=3, gate="mixed"),
    "tp1":    dict(B=1, T=32768, h_qk=16, h_v=16, seed=4, gate="mixed"),
    "tp1_b4": dict(B=4, T=32768, h_qk=16, h_v=16, seed=40, gate="mixed"),
    "long":   dict(B=1, T=262144, h_qk=2, h_v=8, seed=5, gate="mixed", fast_frac=0.5,
                   slow_class="near1", init_std=0.1),
}


def config_inputs(name, **override) -> Inputs:
    kw = dict(CONFIGS[name])
    kw.update(override)
    return make_inputs(name=name, **kw)
