"""C ABI on the CPU: the library loads, exports what include/gdn.h declares,
plans, sizes its workspace and rejects bad arguments before any launch.

No call here reaches a kernel launch: every gdn_fwd / gdn_chunk_prep call is
made with an argument that validation rejects, and planning is given an
explicit CU count so that it never queries a device.
"""
from __future__ import annotations

import ctypes
import math
import os
import re

import pytest

from gated_deltanet_chunked_03_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(B.LIB_PATH),
                                reason="libgdn.so not built (run __graft_entry__.build())")


def lib():
    return B.load_library()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_function():
    names = header_functions()
    assert set(names) == set(B.EXPORTED), (names, B.EXPORTED)
    l = lib()
    for n in names:
        assert hasattr(l, n), n


def test_poison_build_exports_the_same():
    """The LDS-poisoning debug build (built beside libgdn.so) loads and exports
    every declared function; its GPU test compares its results with the
    normal build's."""
    import os
    path = os.path.join(os.path.dirname(B.LIB_PATH), "libgdn_poison.so")
    l = B.load_library(path)
    for n in header_functions():
        assert hasattr(l, n), n


def test_status_strings():
    l = lib()
    for code, name in enumerate(B.STATUS_NAMES):
        assert l.gdn_status_string(code).decode().startswith(name)


def desc(**kw):
    args = dict(B=1, T=32768, h_qk=2, h_v=8, n_cu=256)
    args.update(kw)
    d, keep = B.make_desc(**args)
    return d, keep


def plan(**kw):
    d, keep = desc(**kw)
    return B.plan_desc(d)


# ---------------------------------------------------------------- planner

def n_chunks(t):
    return (t + 63) // 64


def expected_L(lens, h_v, n_cu, lam=1.0, w=6, mode="auto"):
    """The planner rule stated in gdn_api.cpp: among L <= round-half-up(lam sqrt(N_max))
    whose segments times heads cover the CUs (or L = 1), the least
    ceil(segments h_v / CUs) L + L / 2 + (P - 1) / 4, ties to the larger L; AUTO
    keeps sequences whole when sequences x heads already cover the CUs or N_max < 2 (w + 1)."""
    Nm = max(n_chunks(t) for t in lens)
    if mode == "off" or Nm <= 1:
        return max(Nm, 1)
    if mode == "auto" and (len(lens) * h_v >= n_cu or Nm < 2 * (w + 1)):
        return max(Nm, 1)
    L_lam = min(max(1, int(math.floor(lam * math.sqrt(Nm) + 0.5))), Nm)
    segs = lambda L: sum(1 if n_chunks(t) == 0 else -(-n_chunks(t) // L) for t in lens)  # noqa
    best = None
    for L in range(L_lam, 0, -1):
        wg = segs(L) * h_v
        if wg < n_cu and L > 1:
            continue
        cost = -(-wg // n_cu) * L + 0.5 * L + 0.25 * (-(-Nm // L) - 1)
        if best is None or cost < best[0]:
            best = (cost, L)
    return best[1]


@pytest.mark.parametrize("name,B_,T,h_qk,h_v,L", [
    ("tp8", 1, 32768, 2, 8, 16),      # sqrt(512) = 22.6 -> 23; 16 is the largest that fills 256 CUs
    ("tp2", 1, 32768, 8, 24, 16),     # 16 x 24 x 32 segments = three whole rounds (23: 552 workgroups)
    ("tp1", 1, 32768, 16, 16, 16),    # two whole rounds
    ("tp1_b4", 4, 32768, 16, 16, 16),
    ("long", 1, 262144, 2, 8, 43),   # 96 segments x 8 heads = three whole rounds
    ("tiny", 1, 512, 1, 1, 8),        # 8 chunks < 2 (6 + 1): kept whole
])
def test_plan_for_the_workloads(name, B_, T, h_qk, h_v, L):
    p = plan(B=B_, T=T, h_qk=h_qk, h_v=h_v)
    assert p["L"] == L == expected_L([T] * B_, h_v, 256)
    N = n_chunks(T)
    assert p["n_chunks_max"] == N and p["n_chunks_total"] == N * B_
    assert p["P_max"] == -(-N // L) and p["n_segments"] == B_ * p["P_max"]
    assert p["cp_on"] == int(p["P_max"] > 1)
    per_seg = h_v * 128 * 128 * 4
    # the scratch line, then T diag(beta) as fp16 operand images (6 KiB per chunk and value
    # head) and the chunk's gate factors (4 x 64 fp32)
    prep = 8192 + p["n_chunks_total"] * h_v * (6 * 64 * 8 * 2 + 4 * 64 * 4)
    if p["cp_on"]:
        flags = -(-(p["n_segments"] * h_v * 4) // 256) * 256
        # boundary states and H maps (fp32), M maps (fp16 images), boundary flags
        ws_expect = prep + 2 * p["n_segments"] * per_seg + p["n_segments"] * per_seg // 2 + flags
        # the forward's grouped combine (the rule stated in gdn_api.cpp): G boundaries per
        # group when G load1 + (J - 2 + G) load2 + 8 steps come to less than 0.8 of the
        # single chain's P - 1, J = ceil((P - 1) / G), assuming 30 % of the (sequence,
        # head) pairs exact (to the nearest, at least one); load1 = max(1, 16 (J - 1)
        # heads / CUs), load2 = max(1, 8 (J - 1) heads / CUs)
        nb, G_exp = p["P_max"] - 1, 0
        best = 0.8 * nb
        heads = max(1, (B_ * h_v * 3 + 5) // 10)
        for G in range(2, nb):
            J = -(-nb // G)
            if J < 2:
                break
            load1 = max(1.0, 16 * (J - 1) * heads / 256)
            load2 = max(1.0, 8 * (J - 1) * heads / 256)
            steps = G * load1 + (J - 2 + G) * load2 + 8
            if steps < best:
                best, G_exp = steps, G
        assert p["combine_group"] == G_exp
        J_exp = -(-nb // G_exp) if G_exp else 0
        assert p["combine_groups"] == J_exp
        # its composed maps: per (sequence, group, head) CM (fp16) and CH (fp32)
        if G_exp:
            grp = B_ * J_exp * h_v * 128 * 128
            ws_expect += -(-(grp * 2) // 256) * 256 + -(-(grp * 4) // 256) * 256
        assert p["workspace_bytes"] == ws_expect
    else:
        assert p["workspace_bytes"] == prep and p["combine_group"] == 0


def test_plan_options_and_modes():
    assert plan(cp_mode="off")["cp_on"] == 0
    p = plan(lam=0.5)
    assert p["L"] == expected_L([32768], 8, 256, lam=0.5) and p["lambda"] == pytest.approx(0.5)
    # forced modes split even when the heads already cover the CUs
    assert plan(B=4, h_qk=16, h_v=64, cp_mode="auto")["cp_on"] == 0
    assert plan(B=4, h_qk=16, h_v=64, cp_mode="exact")["cp_on"] == 1
    assert plan(warmup_chunks=8)["warmup_chunks"] == 8
    assert plan()["warmup_chunks"] == 6 and plan()["noise_floor"] == pytest.approx(1e-4)


def test_plan_varlen():
    cu = [0, 700, 700, 701, 64 * 20 + 3, 64 * 20 + 3 + 130]
    p = plan(T=cu[-1], h_qk=1, h_v=4, cu_seqlens=cu, n_cu=64, warmup_chunks=2, cp_mode="exact")
    lens = [cu[i + 1] - cu[i] for i in range(len(cu) - 1)]
    L = expected_L(lens, 4, 64, w=2, mode="exact")
    assert p["L"] == L
    assert p["n_chunks_total"] == sum(n_chunks(t) for t in lens)
    assert p["n_segments"] == sum(1 if n_chunks(t) == 0 else -(-n_chunks(t) // L) for t in lens)


@pytest.mark.parametrize("B_,T,h_v,n_cu", [(1, 32768, 8, 256), (1, 4096, 3, 100), (2, 100000, 5, 304),
                                           (1, 262144, 8, 256), (1, 1000, 2, 8)])
def test_plan_fill_property(B_, T, h_v, n_cu):
    """L never exceeds N, and either the segments cover the CUs or L is 1."""
    p = plan(B=B_, T=T, h_qk=1, h_v=h_v, n_cu=n_cu, cp_mode="exact")
    assert 1 <= p["L"] <= max(p["n_chunks_max"], 1)
    assert p["n_segments"] * h_v >= n_cu or p["L"] == 1


# ---------------------------------------------------------------- validation

def call_fwd(d, q=0x1000, k=0x1000, v=0x1000, g=0x1000, beta=0x1000, scale=0.1, s0=None, cu=None,
             out=0x1000, fs=None, ws=None, ws_bytes=0):
    l = lib()
    P = ctypes.c_void_p
    st = l.gdn_fwd(ctypes.byref(d), P(q), P(k), P(v), P(g), P(beta), scale, P(s0) if s0 else None,
                   P(cu) if cu else None, P(out), P(fs) if fs else None, P(ws) if ws else None,
                   ws_bytes, None)
    return st, l.gdn_last_error().decode()


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), "GDN_ERR_BAD_SHAPE"),
    (dict(T=-1), "GDN_ERR_BAD_SHAPE"),
    (dict(h_qk=3, h_v=8), "GDN_ERR_BAD_SHAPE"),
    (dict(d_k=64, d_v=64), "GDN_ERR_UNSUPPORTED_DIM"),
    (dict(io_dtype=7), "GDN_ERR_BAD_DTYPE"),
    (dict(cp_mode=9), "GDN_ERR_BAD_OPTION"),
    (dict(lam=-1.0), "GDN_ERR_BAD_OPTION"),
    (dict(warmup_chunks=9), "GDN_ERR_BAD_OPTION"),
    (dict(noise_floor=1.5), "GDN_ERR_BAD_OPTION"),
    (dict(B=2, cu_seqlens=[0, 10, 20], T=20), "GDN_ERR_BAD_SHAPE"),
    (dict(T=20, cu_seqlens=[0, 15, 10, 20]), "GDN_ERR_BAD_SHAPE"),
    (dict(T=20, cu_seqlens=[0, 10, 19]), "GDN_ERR_BAD_SHAPE"),
    (dict(dv_split=3), "GDN_ERR_BAD_OPTION"),
    (dict(dv_split=2, io_dtype=1), "GDN_ERR_BAD_OPTION"),
    (dict(dv_split=4, cp_mode="exact"), "GDN_ERR_BAD_OPTION"),
    (dict(cp_layout=3), "GDN_ERR_BAD_OPTION"),
    (dict(cp_layout=-1), "GDN_ERR_BAD_OPTION"),
])
def test_bad_descriptor(kw, status):
    d, keep = desc(**kw)
    st, msg = call_fwd(d)
    assert B.STATUS_NAMES[st] == status, msg
    assert msg
    info = B.GdnPlanInfo()
    assert lib().gdn_plan(ctypes.byref(d), ctypes.byref(info)) == st
    assert lib().gdn_fwd_workspace_bytes(ctypes.byref(d)) == 0


def test_null_and_misaligned_pointers():
    d, keep = desc(cp_mode="off")
    assert B.STATUS_NAMES[call_fwd(d, q=0)[0]] == "GDN_ERR_NULL_ARG"
    assert B.STATUS_NAMES[call_fwd(d, out=0)[0]] == "GDN_ERR_NULL_ARG"
    assert B.STATUS_NAMES[call_fwd(d, beta=0)[0]] == "GDN_ERR_NULL_ARG"
    st, msg = call_fwd(d, k=0x1002)
    assert B.STATUS_NAMES[st] == "GDN_ERR_MISALIGNED" and "k" in msg
    assert B.STATUS_NAMES[call_fwd(d, s0=0x1004)[0]] == "GDN_ERR_MISALIGNED"
    # cu_seqlens on the device without the host copy in the descriptor (and vice versa)
    assert B.STATUS_NAMES[call_fwd(d, cu=0x1000)[0]] == "GDN_ERR_NULL_ARG"
    d2, keep2 = desc(T=20, cu_seqlens=[0, 10, 20], cp_mode="off")
    assert B.STATUS_NAMES[call_fwd(d2)[0]] == "GDN_ERR_NULL_ARG"


def test_scale_and_workspace():
    d, keep = desc(cp_mode="off")
    assert B.STATUS_NAMES[call_fwd(d, scale=float("nan"))[0]] == "GDN_ERR_BAD_SCALE"
    assert B.STATUS_NAMES[call_fwd(d, scale=float("inf"))[0]] == "GDN_ERR_BAD_SCALE"
    d, keep = desc()  # CP on: needs a workspace
    need = lib().gdn_fwd_workspace_bytes(ctypes.byref(d))
    assert need > 0
    st, msg = call_fwd(d, ws=0x1000, ws_bytes=need - 1)
    assert B.STATUS_NAMES[st] == "GDN_ERR_WORKSPACE_TOO_SMALL" and str(need) in msg
    st, msg = call_fwd(d, ws=0x1010, ws_bytes=need)
    assert B.STATUS_NAMES[st] == "GDN_ERR_MISALIGNED"


def test_chunk_prep_validation():
    l = lib()
    d, keep = desc(d_k=64)
    P = ctypes.c_void_p
    st = l.gdn_chunk_prep(ctypes.byref(d), P(0x1000), P(0x1000), P(0x1000), P(0x1000), None,
                          P(0x1000), P(0x1000), P(0x1000), None)
    assert B.STATUS_NAMES[st] == "GDN_ERR_UNSUPPORTED_DIM"
    d, keep = desc()
    st = l.gdn_chunk_prep(ctypes.byref(d), P(0x1000), P(0x1000), P(0x1000), P(0x1000), None,
                          None, P(0x1000), P(0x1000), None)
    assert B.STATUS_NAMES[st] == "GDN_ERR_NULL_ARG"


def call_decode(d, q=0x1000, k=0x1000, v=0x1000, g=0x1000, beta=0x1000, scale=0.1, s_in=None, s_out=None,
                out=0x1000):
    l = lib()
    P = ctypes.c_void_p
    st = l.gdn_decode(ctypes.byref(d), P(q), P(k), P(v), P(g), P(beta), scale, P(s_in) if s_in else None,
                      P(s_out) if s_out else None, P(out), None)
    return st, l.gdn_last_error().decode()


def test_decode_validation():
    """gdn_decode rejects bad descriptors and pointers before any launch."""
    d, keep = desc(B=4, T=1, d_k=64, d_v=64)
    assert B.STATUS_NAMES[call_decode(d)[0]] == "GDN_ERR_UNSUPPORTED_DIM"
    d, keep = desc(T=20, cu_seqlens=[0, 10, 20])
    st, msg = call_decode(d)
    assert B.STATUS_NAMES[st] == "GDN_ERR_BAD_SHAPE" and "cu_seqlens" in msg
    d, keep = desc(B=4, T=1)
    assert B.STATUS_NAMES[call_decode(d, q=0)[0]] == "GDN_ERR_NULL_ARG"
    assert B.STATUS_NAMES[call_decode(d, out=0)[0]] == "GDN_ERR_NULL_ARG"
    assert B.STATUS_NAMES[call_decode(d, v=0x1008)[0]] == "GDN_ERR_MISALIGNED"
    assert B.STATUS_NAMES[call_decode(d, s_in=0x1004)[0]] == "GDN_ERR_MISALIGNED"
    assert B.STATUS_NAMES[call_decode(d, scale=float("nan"))[0]] == "GDN_ERR_BAD_SCALE"
    # states: the same buffer is allowed, a partial overlap is not
    st, msg = call_decode(d, s_in=0x100000, s_out=0x100000 + 65536)
    assert B.STATUS_NAMES[st] == "GDN_ERR_BAD_SHAPE" and "overlap" in msg


def call_bwd(d, q=0x1000, k=0x1000, v=0x1000, g=0x1000, beta=0x1000, scale=0.1, s0=None, cu=None,
             dout=0x1000, dfin=None, dq=0x1000, dk=0x1000, dv=0x1000, dg=0x1000, dbeta=0x1000, dinit=None,
             ws=0x1000, ws_bytes=1 << 40):
    l = lib()
    P = ctypes.c_void_p
    opt = lambda x: P(x) if x else None  # noqa: E731
    st = l.gdn_bwd(ctypes.byref(d), P(q), P(k), P(v), P(g), P(beta), scale, opt(s0), opt(cu), opt(dout),
                   opt(dfin), opt(dq), opt(dk), opt(dv), opt(dg), opt(dbeta), opt(dinit), opt(ws), ws_bytes, None)
    return st, l.gdn_last_error().decode()


def test_bwd_validation():
    """gdn_bwd rejects bad arguments before any launch (dtype; every gradient
    output and d_out required; workspace size and alignment)."""
    d, keep = desc(io_dtype=7)
    assert B.STATUS_NAMES[call_bwd(d)[0]] == "GDN_ERR_BAD_DTYPE"
    # fp32 inputs: the workspace also holds their bf16 copies (q, k: 2 x 256 B per
    # token and query/key head; v, d_out: 2 x 256 B per token and value head)
    d16, keep16 = desc()
    d32, keep32 = desc(io_dtype=B.GDN_F32)
    n16 = lib().gdn_bwd_workspace_bytes(ctypes.byref(d16))
    n32 = lib().gdn_bwd_workspace_bytes(ctypes.byref(d32))
    assert n32 >= n16 + 2 * 256 * d32.B * d32.T * (d32.h_qk + d32.h_v)
    st, msg = call_bwd(d32, ws_bytes=n32 - 1)
    assert B.STATUS_NAMES[st] == "GDN_ERR_WORKSPACE_TOO_SMALL" and str(n32) in msg
    d, keep = desc(d_k=64, d_v=64)
    assert B.STATUS_NAMES[call_bwd(d)[0]] == "GDN_ERR_UNSUPPORTED_DIM"
    d, keep = desc()
    for kw in ("dout", "dq", "dk", "dv", "dg", "dbeta", "q"):
        st, msg = call_bwd(d, **{kw: 0})
        assert B.STATUS_NAMES[st] == "GDN_ERR_NULL_ARG", (kw, msg)
    assert B.STATUS_NAMES[call_bwd(d, dg=0x1002)[0]] == "GDN_ERR_MISALIGNED"
    assert B.STATUS_NAMES[call_bwd(d, scale=float("inf"))[0]] == "GDN_ERR_BAD_SCALE"
    need = lib().gdn_bwd_workspace_bytes(ctypes.byref(d))
    assert need > lib().gdn_fwd_workspace_bytes(ctypes.byref(d))
    st, msg = call_bwd(d, ws_bytes=need - 1)
    assert B.STATUS_NAMES[st] == "GDN_ERR_WORKSPACE_TOO_SMALL" and str(need) in msg
    assert B.STATUS_NAMES[call_bwd(d, ws=0x1010, ws_bytes=need)[0]] == "GDN_ERR_MISALIGNED"
    d2, keep2 = desc(T=20, cu_seqlens=[0, 10, 20])
    assert B.STATUS_NAMES[call_bwd(d2)[0]] == "GDN_ERR_NULL_ARG"   # device cu_seqlens missing


def test_calibrate_lambda_validation():
    """gdn_calibrate_lambda checks its candidates and the workspace before running anything."""
    l = lib()
    P = ctypes.c_void_p
    d, keep = desc()
    best = ctypes.c_float()

    def call(lams, n=None, reps=3, ws_bytes=1 << 40, best_p=True):
        arr = (ctypes.c_float * max(len(lams), 1))(*lams)
        st = l.gdn_calibrate_lambda(ctypes.byref(d), P(0x1000), P(0x1000), P(0x1000), P(0x1000), P(0x1000), 0.1,
                                    None, P(0x1000), P(0x1000), ws_bytes, arr, len(lams) if n is None else n,
                                    reps, None, None, ctypes.byref(best) if best_p else None)
        return B.STATUS_NAMES[st], l.gdn_last_error().decode()

    assert call([1.0], n=0)[0] == "GDN_ERR_BAD_OPTION"
    assert call([1.0], reps=0)[0] == "GDN_ERR_BAD_OPTION"
    assert call([1.0, -2.0])[0] == "GDN_ERR_BAD_OPTION"
    assert call([float("nan")])[0] == "GDN_ERR_BAD_OPTION"
    assert call([1.0], best_p=False)[0] == "GDN_ERR_NULL_ARG"
    need = max(plan(lam=x)["workspace_bytes"] for x in (0.5, 2.0))
    st, msg = call([0.5, 2.0], ws_bytes=need - 1)
    assert st == "GDN_ERR_WORKSPACE_TOO_SMALL" and str(need) in msg


def test_profile_read_without_profiled_call():
    l = lib()
    ms = (ctypes.c_float * 5)()
    assert B.STATUS_NAMES[l.gdn_profile_read(ms)] == "GDN_ERR_BAD_OPTION"
    assert B.STATUS_NAMES[l.gdn_profile_read(None)] == "GDN_ERR_NULL_ARG"


def test_python_binding_rejects_host_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(1, 64, 1, 128)
    g = torch.zeros(1, 64, 1)
    with pytest.raises(ValueError):
        B.fwd(x, x, x, g, g)


def test_plan_cp_layout():
    """Boundary preprocessing layout: the planner takes two workgroups per
    exact boundary (2) when every boundary pair fits on the CUs at once (TP8:
    32 x 8 on 256 CUs; with cp_mode EXACT every pair counts twice), else one
    (1: TP2, TP1, long); a forced layout is kept; 0 without a split or with
    fp32 inputs."""
    assert B.plan(1, 32768, 2, 8, n_cu=256)["cp_layout"] == 2
    for args in [(1, 32768, 8, 24), (1, 32768, 16, 16), (1, 262144, 2, 8)]:
        assert B.plan(*args, n_cu=256)["cp_layout"] == 1, args
    for lay in (1, 2):
        assert B.plan(1, 32768, 2, 8, n_cu=256, cp_layout=lay)["cp_layout"] == lay
        assert B.plan(1, 32768, 16, 16, n_cu=256, cp_layout=lay)["cp_layout"] == lay
    assert B.plan(1, 32768, 2, 8, n_cu=256, cp_mode="exact")["cp_layout"] == 1   # 2 x 256 workgroups
    assert B.plan(1, 32768, 2, 8, n_cu=256, cp_mode="off")["cp_layout"] == 0
    assert B.plan(1, 32768, 2, 8, n_cu=256, io_dtype=B.GDN_F32)["cp_layout"] == 0


def test_plan_column_split():
    """d_v column blocks: forced (1, 2, 4) runs without segments; AUTO takes
    them only where they fill the CUs and the estimate beats the segment split
    (short sequences, sequences x heads = half the CUs), never for fp32 inputs,
    and keeps the split at the TP shapes (measured faster there)."""
    for s_dv in (1, 2, 4):
        p = B.plan(1, 32768, 2, 8, n_cu=256, dv_split=s_dv)
        assert p["dv_split"] == s_dv and (p["cp_on"] == 0 or s_dv == 1)
    p = B.plan(16, 896, 8, 8, n_cu=256)
    assert (p["cp_on"], p["dv_split"], p["L"]) == (0, 2, 14)
    p = B.plan(16, 896, 8, 8, n_cu=256, io_dtype=B.GDN_F32)
    assert p["cp_on"] == 1 and p["dv_split"] == 1
    for args in [(1, 32768, 2, 8), (4, 32768, 16, 16), (1, 32768, 16, 16)]:
        p = B.plan(*args, n_cu=256)
        assert p["dv_split"] == 1 and p["cp_on"] == 1, args
    # forced column split with cp_mode OFF; workspace without the split's arrays
    p0 = B.plan(1, 32768, 2, 8, n_cu=256, cp_mode="off")
    p4 = B.plan(1, 32768, 2, 8, n_cu=256, dv_split=4)
    assert p4["workspace_bytes"] == p0["workspace_bytes"]
