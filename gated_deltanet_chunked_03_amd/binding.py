"""ctypes binding of ``libgdn.so`` (include/gdn.h): argument marshalling only.

Every step of the forward runs in the HIP kernels behind the C ABI; torch only
supplies device memory and the current stream. If the library has not been
built, calls raise instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import math
import os
import threading
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "_build", "libgdn.so")

GDN_OK = 0
STATUS_NAMES = ["GDN_OK", "GDN_ERR_NULL_ARG", "GDN_ERR_BAD_SHAPE", "GDN_ERR_UNSUPPORTED_DIM",
                "GDN_ERR_BAD_DTYPE", "GDN_ERR_MISALIGNED", "GDN_ERR_BAD_SCALE",
                "GDN_ERR_WORKSPACE_TOO_SMALL", "GDN_ERR_BAD_OPTION", "GDN_ERR_HIP"]
CP_MODES = {"auto": 0, "off": 1, "exact": 2, "warmup": 3}
GDN_BF16, GDN_F32 = 0, 1

EXPORTED = ["gdn_plan", "gdn_fwd_workspace_bytes", "gdn_fwd", "gdn_fwd_noalloc", "gdn_fwd_debug", "gdn_chunk_prep",
            "gdn_decode", "gdn_bwd_workspace_bytes", "gdn_bwd", "gdn_calibrate_lambda", "gdn_profile_enable", "gdn_profile_read", "gdn_status_string", "gdn_last_error"]


class GdnDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("h_qk", ctypes.c_int32),
                ("h_v", ctypes.c_int32), ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("n_seqs", ctypes.c_int32), ("host_cu_seqlens", ctypes.POINTER(ctypes.c_int32)),
                ("io_dtype", ctypes.c_int32), ("cp_mode", ctypes.c_int32),
                ("lambda_", ctypes.c_float), ("warmup_chunks", ctypes.c_int32),
                ("noise_floor", ctypes.c_float), ("n_cu", ctypes.c_int32), ("dv_split", ctypes.c_int32),
                ("cp_layout", ctypes.c_int32)]


class GdnPlanInfo(ctypes.Structure):
    _fields_ = [("chunk", ctypes.c_int32), ("n_chunks_total", ctypes.c_int32),
                ("n_chunks_max", ctypes.c_int32), ("cp_on", ctypes.c_int32), ("L", ctypes.c_int32),
                ("n_segments", ctypes.c_int32), ("P_max", ctypes.c_int32),
                ("warmup_chunks", ctypes.c_int32), ("n_cu", ctypes.c_int32),
                ("lambda_", ctypes.c_float), ("noise_floor", ctypes.c_float),
                ("workspace_bytes", ctypes.c_size_t), ("combine_group", ctypes.c_int32),
                ("combine_groups", ctypes.c_int32), ("dv_split", ctypes.c_int32),
                ("cp_layout", ctypes.c_int32)]

    def as_dict(self):
        d = {f: getattr(self, f) for f, _ in self._fields_}
        d["lambda"] = d.pop("lambda_")
        return d


class GDNError(RuntimeError):
    def __init__(self, status, detail):
        name = STATUS_NAMES[status] if 0 <= status < len(STATUS_NAMES) else f"status {status}"
        super().__init__(f"{name}: {detail}")
        self.status = status


_lib = None
_lock = threading.Lock()


def load_library(path: Optional[str] = None):
    """Load libgdn.so (built in-tree by gated_deltanet_chunked_03_amd.build)."""
    global _lib
    with _lock:
        if _lib is not None and path is None:
            return _lib
        p = path or LIB_PATH
        if not os.path.exists(p):
            raise RuntimeError(f"HIP library {p} is not built; run "
                               "`python -m gated_deltanet_chunked_03_amd.build` first")
        lib = ctypes.CDLL(p)
        P = ctypes.c_void_p
        S = ctypes.c_int
        lib.gdn_plan.argtypes = [ctypes.POINTER(GdnDesc), ctypes.POINTER(GdnPlanInfo)]
        lib.gdn_plan.restype = S
        lib.gdn_fwd_workspace_bytes.argtypes = [ctypes.POINTER(GdnDesc)]
        lib.gdn_fwd_workspace_bytes.restype = ctypes.c_size_t
        fwd_args = [ctypes.POINTER(GdnDesc), P, P, P, P, P, ctypes.c_float, P, P, P, P, P,
                    ctypes.c_size_t, P]
        lib.gdn_fwd.argtypes = fwd_args
        lib.gdn_fwd.restype = S
        lib.gdn_fwd_noalloc.argtypes = fwd_args[:11] + [P]
        lib.gdn_fwd_noalloc.restype = S
        lib.gdn_fwd_debug.argtypes = fwd_args + [P, P]
        lib.gdn_fwd_debug.restype = S
        lib.gdn_chunk_prep.argtypes = [ctypes.POINTER(GdnDesc), P, P, P, P, P, P, P, P, P]
        lib.gdn_chunk_prep.restype = S
        lib.gdn_decode.argtypes = [ctypes.POINTER(GdnDesc), P, P, P, P, P, ctypes.c_float, P, P, P, P]
        lib.gdn_decode.restype = S
        lib.gdn_bwd_workspace_bytes.argtypes = [ctypes.POINTER(GdnDesc)]
        lib.gdn_bwd_workspace_bytes.restype = ctypes.c_size_t
        lib.gdn_bwd.argtypes = [ctypes.POINTER(GdnDesc), P, P, P, P, P, ctypes.c_float, P, P, P, P,
                                P, P, P, P, P, P, P, ctypes.c_size_t, P]
        lib.gdn_bwd.restype = S
        lib.gdn_calibrate_lambda.argtypes = [ctypes.POINTER(GdnDesc), P, P, P, P, P, ctypes.c_float, P, P, P,
                                             ctypes.c_size_t, P, ctypes.c_int32, ctypes.c_int32, P, P, P]
        lib.gdn_calibrate_lambda.restype = S
        lib.gdn_profile_enable.argtypes = [ctypes.c_int]
        lib.gdn_profile_enable.restype = S
        lib.gdn_profile_read.argtypes = [ctypes.POINTER(ctypes.c_float)]
        lib.gdn_profile_read.restype = S
        lib.gdn_status_string.argtypes = [S]
        lib.gdn_status_string.restype = ctypes.c_char_p
        lib.gdn_last_error.argtypes = []
        lib.gdn_last_error.restype = ctypes.c_char_p
        if path is None:
            _lib = lib
        return lib


def _check(lib, status):
    if status != GDN_OK:
        raise GDNError(status, lib.gdn_last_error().decode())


def make_desc(B, T, h_qk, h_v, d_k=128, d_v=128, io_dtype=GDN_BF16, cu_seqlens=None,
              cp_mode="auto", lam=0.0, warmup_chunks=0, noise_floor=0.0, n_cu=0, dv_split=0, cp_layout=0):
    """Descriptor plus the host cu_seqlens buffer it points to (keep both alive)."""
    d = GdnDesc()
    d.B, d.T, d.h_qk, d.h_v, d.d_k, d.d_v = B, T, h_qk, h_v, d_k, d_v
    host_cu = None
    if cu_seqlens is not None:
        vals = [int(x) for x in cu_seqlens]
        host_cu = (ctypes.c_int32 * len(vals))(*vals)
        d.host_cu_seqlens = ctypes.cast(host_cu, ctypes.POINTER(ctypes.c_int32))
        d.n_seqs = len(vals) - 1
    else:
        d.n_seqs = B
    d.io_dtype = io_dtype
    d.cp_mode = CP_MODES[cp_mode] if isinstance(cp_mode, str) else int(cp_mode)
    d.lambda_, d.warmup_chunks, d.noise_floor, d.n_cu = lam, warmup_chunks, noise_floor, n_cu
    d.dv_split = dv_split
    d.cp_layout = cp_layout
    return d, host_cu


def plan_desc(desc):
    lib = load_library()
    info = GdnPlanInfo()
    _check(lib, lib.gdn_plan(ctypes.byref(desc), ctypes.byref(info)))
    return info.as_dict()


def plan(B, T, h_qk, h_v, d_k=128, d_v=128, io_dtype=GDN_BF16, cu_seqlens=None, cp_mode="auto",
         lam=0.0, warmup_chunks=0, noise_floor=0.0, n_cu=0, dv_split=0, cp_layout=0):
    """Host-only planning (n_cu=0 queries the current device)."""
    d, keep = make_desc(B, T, h_qk, h_v, d_k, d_v, io_dtype, cu_seqlens, cp_mode, lam, warmup_chunks,
                        noise_floor, n_cu, dv_split, cp_layout)
    out = plan_desc(d)
    del keep
    return out


# ---------------------------------------------------------------------------- torch side

def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _req(t, name, dtype, device, shape=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _prepare(q, k, v, g, beta, cu_seqlens):
    torch = _torch()
    if q.dim() != 4:
        raise ValueError("q must be [B, T, h_qk, d_k]")
    B, T, h_qk, d_k = q.shape
    h_v, d_v = v.shape[2], v.shape[3]
    if q.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("q, k, v must be bfloat16 or float32")
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU device")
    _req(q, "q", q.dtype, dev)
    _req(k, "k", q.dtype, dev, (B, T, h_qk, d_k))
    _req(v, "v", q.dtype, dev, (B, T, h_v, d_v))
    _req(g, "g", torch.float32, dev, (B, T, h_v))
    _req(beta, "beta", torch.float32, dev, (B, T, h_v))
    cu_dev, cu_host = None, None
    if cu_seqlens is not None:
        if isinstance(cu_seqlens, torch.Tensor):
            cu_host = [int(x) for x in cu_seqlens.tolist()]   # one host sync if on the GPU
        else:
            cu_host = [int(x) for x in cu_seqlens]
        cu_dev = torch.tensor(cu_host, dtype=torch.int32, device=dev)
    io = GDN_BF16 if q.dtype == torch.bfloat16 else GDN_F32
    return B, T, h_qk, h_v, d_k, d_v, io, cu_dev, cu_host


def fwd(q, k, v, g, beta, scale=None, initial_state=None, output_final_state=True,
        cu_seqlens=None, cp_mode="auto", lam=0.0, warmup_chunks=0, noise_floor=0.0, n_cu=0,
        workspace=None, out=None, final_state=None, debug=False, dv_split=0, cp_layout=0):
    """Gated DeltaNet chunked-prefill forward on the GPU.

    q, k: [B, T, h_qk, 128]; v: [B, T, h_v, 128] (bf16 or fp32, same dtype);
    g (= log alpha <= 0), beta: [B, T, h_v] fp32; initial_state: [n_seqs, h_v, 128, 128]
    fp32 or None; cu_seqlens: packed sequence offsets (B == 1) as a list or tensor.
    Returns (o, final_state); with debug=True also a dict with the plan, the
    segment initial states and the per-head path summary.
    """
    torch = _torch()
    B, T, h_qk, h_v, d_k, d_v, io, cu_dev, cu_host = _prepare(q, k, v, g, beta, cu_seqlens)
    dev = q.device
    n_seqs = B if cu_host is None else len(cu_host) - 1
    if scale is None:
        scale = 1.0 / math.sqrt(d_k)
    if initial_state is not None:
        _req(initial_state, "initial_state", torch.float32, dev, (n_seqs, h_v, d_k, d_v))
    desc, keep = make_desc(B, T, h_qk, h_v, d_k, d_v, io, cu_host, cp_mode, lam, warmup_chunks,
                           noise_floor, n_cu, dv_split, cp_layout)
    lib = load_library()
    info = plan_desc(desc)
    if out is None:
        out = torch.empty_like(v)
    else:
        _req(out, "out", v.dtype, dev, tuple(v.shape))
    fs = None
    if output_final_state:
        if final_state is None:
            fs = torch.empty((n_seqs, h_v, d_k, d_v), dtype=torch.float32, device=dev)
        else:
            _req(final_state, "final_state", torch.float32, dev, (n_seqs, h_v, d_k, d_v))
            fs = final_state
    ws_bytes = info["workspace_bytes"]
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    args = [ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale),
            _ptr(initial_state), _ptr(cu_dev), _ptr(out), _ptr(fs), _ptr(workspace),
            workspace.numel() * workspace.element_size(), stream]
    if not debug:
        _check(lib, lib.gdn_fwd(*args))
        del keep
        return out, fs
    seg = torch.empty((info["n_segments"], h_v, d_k, d_v), dtype=torch.float32, device=dev)
    path = torch.empty((n_seqs, h_v), dtype=torch.int32, device=dev)
    _check(lib, lib.gdn_fwd_debug(*args, _ptr(seg), _ptr(path)))
    del keep
    return out, fs, {"plan": info, "seg_state": seg, "path": path}


def fwd_noalloc(q, k, v, g, beta, scale=None, initial_state=None, output_final_state=True,
                cu_seqlens=None, cp_mode="auto", lam=0.0, warmup_chunks=0, noise_floor=0.0, n_cu=0,
                out=None, final_state=None, dv_split=0, cp_layout=0):
    """``fwd`` through gdn_fwd_noalloc: the library's per-device scratch array
    serves as the workspace (descriptors needing more than
    NOALLOC_SCRATCH_BYTES raise). Calls that overlap on one device race."""
    torch = _torch()
    B, T, h_qk, h_v, d_k, d_v, io, cu_dev, cu_host = _prepare(q, k, v, g, beta, cu_seqlens)
    dev = q.device
    n_seqs = B if cu_host is None else len(cu_host) - 1
    if scale is None:
        scale = 1.0 / math.sqrt(d_k)
    if initial_state is not None:
        _req(initial_state, "initial_state", torch.float32, dev, (n_seqs, h_v, d_k, d_v))
    desc, keep = make_desc(B, T, h_qk, h_v, d_k, d_v, io, cu_host, cp_mode, lam, warmup_chunks,
                           noise_floor, n_cu, dv_split, cp_layout)
    lib = load_library()
    if out is None:
        out = torch.empty_like(v)
    else:
        _req(out, "out", v.dtype, dev, tuple(v.shape))
    fs = None
    if output_final_state:
        if final_state is None:
            fs = torch.empty((n_seqs, h_v, d_k, d_v), dtype=torch.float32, device=dev)
        else:
            _req(final_state, "final_state", torch.float32, dev, (n_seqs, h_v, d_k, d_v))
            fs = final_state
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    _check(lib, lib.gdn_fwd_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                    float(scale), _ptr(initial_state), _ptr(cu_dev), _ptr(out), _ptr(fs),
                                    stream))
    del keep
    return out, fs


NOALLOC_SCRATCH_BYTES = 80 << 20   # GDN_NOALLOC_SCRATCH_BYTES of include/gdn.h


def profile_enable(on=True):
    """Record HIP events around each kernel of later fwd calls (measurement only)."""
    lib = load_library()
    _check(lib, lib.gdn_profile_enable(1 if on else 0))


def profile_read():
    """Milliseconds of the last profiled fwd call: dict prep, cp_prep, cp_combine, fwd, total."""
    lib = load_library()
    ms = (ctypes.c_float * 5)()
    _check(lib, lib.gdn_profile_read(ms))
    return {"prep": ms[0], "cp_prep": ms[1], "cp_combine": ms[2], "fwd": ms[3], "total": ms[4]}


def chunk_gated_delta_rule(q, k, v, g, beta, scale=None, initial_state=None,
                           output_final_state=False, cu_seqlens=None):
    """FLA-style argument order (q, k, v, g, beta, scale, initial_state,
    output_final_state, cu_seqlens) -> (o, final_state or None)."""
    return fwd(q, k, v, g, beta, scale=scale, initial_state=initial_state,
               output_final_state=output_final_state, cu_seqlens=cu_seqlens)


def bwd(q, k, v, g, beta, d_out, scale=None, initial_state=None, d_final_state=None, cu_seqlens=None,
        cp_mode="auto", lam=0.0, warmup_chunks=0, noise_floor=0.0, n_cu=0, workspace=None,
        want_d_initial=True):
    """Gradients of ``fwd``: given d_out (like v) and optionally d_final_state
    ([n_seqs, h_v, 128, 128] fp32), returns a dict with dq, dk (like q), dv
    (like v), dg, dbeta (like g) and d_initial ([n_seqs, h_v, 128, 128] fp32, or
    None when want_d_initial is False). The forward runs again inside, with the
    same plan options as ``fwd``. fp32 q, k, v and d_out are rounded once to
    bf16 inside; their gradients come back in fp32."""
    torch = _torch()
    B, T, h_qk, h_v, d_k, d_v, io, cu_dev, cu_host = _prepare(q, k, v, g, beta, cu_seqlens)
    dev = q.device
    n_seqs = B if cu_host is None else len(cu_host) - 1
    if scale is None:
        scale = 1.0 / math.sqrt(d_k)
    _req(d_out, "d_out", v.dtype, dev, tuple(v.shape))
    sshape = (n_seqs, h_v, d_k, d_v)
    if initial_state is not None:
        _req(initial_state, "initial_state", torch.float32, dev, sshape)
    if d_final_state is not None:
        _req(d_final_state, "d_final_state", torch.float32, dev, sshape)
    desc, keep = make_desc(B, T, h_qk, h_v, d_k, d_v, io, cu_host, cp_mode, lam, warmup_chunks,
                           noise_floor, n_cu)
    lib = load_library()
    plan_desc(desc)   # raises on an invalid descriptor
    need = lib.gdn_bwd_workspace_bytes(ctypes.byref(desc))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    out = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
               dg=torch.empty_like(g), dbeta=torch.empty_like(beta),
               d_initial=torch.empty(sshape, dtype=torch.float32, device=dev) if want_d_initial else None)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    _check(lib, lib.gdn_bwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale),
                            _ptr(initial_state), _ptr(cu_dev), _ptr(d_out), _ptr(d_final_state),
                            _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dg"]),
                            _ptr(out["dbeta"]), _ptr(out["d_initial"]), _ptr(workspace),
                            workspace.numel() * workspace.element_size(), stream))
    del keep
    return out


def calibrate_lambda(q, k, v, g, beta, lambdas=(0.5, 0.75, 1.0, 1.5, 2.0), reps=3, scale=None, cu_seqlens=None,
                     cp_mode="auto", warmup_chunks=0, noise_floor=0.0, n_cu=0):
    """Time the forward on these inputs for each candidate lambda (L = lambda sqrt(N))
    and return (best_lambda, {lambda: mean ms per forward}). Synchronises the host."""
    torch = _torch()
    B, T, h_qk, h_v, d_k, d_v, io, cu_dev, cu_host = _prepare(q, k, v, g, beta, cu_seqlens)
    dev = q.device
    if scale is None:
        scale = 1.0 / math.sqrt(d_k)
    lib = load_library()
    need = 256
    for lam in lambdas:
        desc, keep = make_desc(B, T, h_qk, h_v, d_k, d_v, io, cu_host, cp_mode, float(lam), warmup_chunks,
                               noise_floor, n_cu)
        need = max(need, plan_desc(desc)["workspace_bytes"])
    desc, keep = make_desc(B, T, h_qk, h_v, d_k, d_v, io, cu_host, cp_mode, 0.0, warmup_chunks, noise_floor, n_cu)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    out = torch.empty_like(v)
    lam_arr = (ctypes.c_float * len(lambdas))(*[float(x) for x in lambdas])
    ms = (ctypes.c_float * len(lambdas))()
    best = ctypes.c_float()
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    _check(lib, lib.gdn_calibrate_lambda(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                         float(scale), _ptr(cu_dev), _ptr(out), _ptr(ws), need, lam_arr,
                                         len(lambdas), int(reps), stream, ms, ctypes.byref(best)))
    del keep
    return best.value, {float(l): ms[i] for i, l in enumerate(lambdas)}


def decode(q, k, v, g, beta, state, scale=None, out=None, state_out=None, inplace=False):
    """Recurrent decode continuing from ``state``: B rows of T tokens (T = 1
    for one generated token each), same layouts as ``fwd``; state is
    [B, h_v, 128, 128] fp32 or None (zeros). Returns (o, new_state); with
    inplace=True the new state overwrites ``state``."""
    torch = _torch()
    B, T, h_qk, h_v, d_k, d_v, io, _, _ = _prepare(q, k, v, g, beta, None)
    dev = q.device
    if scale is None:
        scale = 1.0 / math.sqrt(d_k)
    if state is not None:
        _req(state, "state", torch.float32, dev, (B, h_v, d_k, d_v))
    if inplace:
        if state is None:
            raise ValueError("inplace=True needs a state")
        state_out = state
    elif state_out is None:
        state_out = torch.empty((B, h_v, d_k, d_v), dtype=torch.float32, device=dev)
    else:
        _req(state_out, "state_out", torch.float32, dev, (B, h_v, d_k, d_v))
    if out is None:
        out = torch.empty_like(v)
    else:
        _req(out, "out", v.dtype, dev, tuple(v.shape))
    desc, keep = make_desc(B, T, h_qk, h_v, d_k, d_v, io)
    lib = load_library()
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    _check(lib, lib.gdn_decode(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                               float(scale), _ptr(state), _ptr(state_out), _ptr(out), stream))
    del keep
    return out, state_out


def chunk_prep(k, v, g, beta, cu_seqlens=None):
    """Low-level chunk preparation: (gamma [n_chunks, h_v, 64], W [n_chunks, h_v, 64, 128],
    U [n_chunks, h_v, 64, 128]) in fp32."""
    torch = _torch()
    B, T, h_qk, h_v, d_k, d_v, io, cu_dev, cu_host = _prepare(k, k, v, g, beta, cu_seqlens)
    desc, keep = make_desc(B, T, h_qk, h_v, d_k, d_v, io, cu_host, "off", n_cu=1)
    lib = load_library()
    info = plan_desc(desc)
    n = info["n_chunks_total"]
    dev = k.device
    gam = torch.empty((n, h_v, 64), dtype=torch.float32, device=dev)
    W = torch.empty((n, h_v, 64, d_k), dtype=torch.float32, device=dev)
    U = torch.empty((n, h_v, 64, d_v), dtype=torch.float32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    _check(lib, lib.gdn_chunk_prep(ctypes.byref(desc), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                   _ptr(cu_dev), _ptr(gam), _ptr(W), _ptr(U), stream))
    del keep
    return gam, W, U
