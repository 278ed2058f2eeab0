#!/usr/bin/env python3
"""Benchmark: Gated DeltaNet chunked-prefill forward on one MI355X.

One step = one call of the library's forward (k_prep, k_cp_prep16, k_combine16
and the fused forward kernel k_fwd_ws) over one batch of seeded synthetic input
already resident in HBM. Before every step a 1 GiB fill evicts the L2 caches
and the 256 MB Infinity Cache (outside the measured interval); each step's GPU
time comes from HIP events on the stream around the step's four eager
launches. A second pass with events between the kernels gives the per-kernel
split; with --graph the step is also replayed from a HIP graph of the same
launches (each replay first checked bit for bit against the eager result) and
timed. The default workload is the TP8-shaped prompt (B=1, T=32768, h_qk=2,
h_v=8, d=128, chunk 64, bf16 inputs).

Prints one JSON line. Besides the contract fields it carries:
  roofline      the whole step's algorithmic HBM bytes / ms_per_step (headline),
                with the dominant kernel's own figure under "kernel" and the
                summed counter traffic of the step's kernels
  mfma          the step's algorithmic matrix work / ms_per_step against the
                dense fp16/bf16 peak
  step_ms_stats median, p10 and p90 of the timed steps
  gpu_clock_mhz the shader clock sampled from sysfs while the timed steps ran
  cpu_baseline  the fp64 CPU oracle timed on the host cores on a token prefix
                (threads used, host core count and CPU model stated)
  parity        GPU output vs that oracle on the same prefix
  boundary_state_error  per value head: the largest relative error of the
                segment initial states the forward used (warm-up or exact)
                against the oracle's states at those boundaries
  backward      the backward pass (gdn_bwd) on the same workload: time per call, bytes,
                matrix work of its chunk-gradient kernel, parity on a token prefix vs the fp64
                backward oracle
  decode        the one-token recurrent decode (gdn_decode) over 256 rows at the TP8 head
                counts: time per call, HBM roofline, outputs and states vs the oracle
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GDN fwd ms & tokens/s at B=1,T=32768 per head config; % MFMA/HBM roofline"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
CSRC = os.path.join(ROOT, "gated_deltanet_chunked_03_amd", "csrc")
# the sources the forward and decode kernels are built from; measured counter
# figures below are valid only for sources with this combined hash
KERNEL_SRCS = [os.path.join(CSRC, f) for f in ("gdn_device.h", "gdn_internal.h", "gdn_kernels.hip",
                                               "gdn_fwd16.hip")]
# HBM bytes per launch of each forward kernel on the tp8 workload (AutoCP, default lambda) and
# of k_decode on the 256-row decode, from rocprofv3 FETCH_SIZE / WRITE_SIZE passes scaled by a
# 512 MiB copy's counts (profiles/forward_kernels_tp8.md, decode_k_decode_256rows.md); None
# until taken for the current sources.
MEASURED_TRAFFIC = {"sha256": "664e70c7552fd5037bd5794484bc80a6623fbd8103e8fc403eff8a24b3149450",
                    # bytes read, written per launch (keys as the per-kernel timings; cp_combine
                    # is the grouped combine's two launches)
                    "tp8": {"per_kernel": {"prep": [19861124, 29393888], "cp_prep": [47348275, 18219008], "cp_combine": [16714197, 5439488], "fwd": [146601421, 67633152]},
                            "dominant": "fwd",
                            # MfmaFlopsF16 + MfmaFlopsBF16 of the step's kernels per step
                            "mfma_flops": 53763000000},
                    "decode256": {"read": 135138864, "write": 134953632}}
# The pages' own per-forward times for 1 x 32768 tokens on an H200 (other hardware; context).
PAGES_MS = {"tp8": 0.310, "tp4": 0.486, "tp2": 0.659, "tp1": 0.493}
MFMA_PEAK_TFLOPS = 2500.0    # MI355X dense fp16 / bf16 matrix peak
DOMINANT_KERNEL = "fwd"      # the fused forward kernel: the step's longest launch


def sources_sha256():
    h = hashlib.sha256()
    for f in KERNEL_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def algorithmic_bytes(B, T, h_qk, h_v, d=128, e_io=2, initial=False, final=True, n_seqs=None):
    """What the forward must move: q, k (per query/key head), v, out (per value
    head), g and beta, plus the states it reads and writes."""
    n_seqs = B if n_seqs is None else n_seqs
    per_token = 2 * h_qk * d * e_io + 2 * h_v * d * e_io + 8 * h_v
    return B * T * per_token + (int(initial) + int(final)) * n_seqs * h_v * d * d * 4


def algorithmic_flops(B, T, h_qk, h_v, d=128, C=64):
    """Per token and value head: 6 d^2 (W S, Q S, K^T V'), C (d + 2 d) (triangular
    T X for W and U, causal P V'), 2 C d h_qk/h_v (K K^T and Q K^T lower halves,
    shared by the head group), 2 C^2 / 3 (64 x 64 triangular inverse)."""
    per = 6 * d * d + C * (d + 2 * d) + 2 * C * d * h_qk / h_v + 2 * C * C / 3
    return B * T * h_v * per


def decode_bytes(rows, h_qk, h_v, d=128, e_io=2):
    """What one decode call must move per row: its state read and written
    (fp32 d x d per value head) plus one token's q, k, v, out, g and beta."""
    return rows * (2 * h_v * d * d * 4 + 2 * h_qk * d * e_io + 2 * h_v * d * e_io + 8 * h_v)


BWD_KERNEL_FLOPS = {
    # useful multiply-adds x 2 per (chunk, value head) of the chunk-gradient kernel: three
    # 64x128x128 products (dO S^T, V' dSn^T, dY S^T), seven 64x64x128 (dP, dT, K K^T, Psi K,
    # Psi^T Q, G K, G^T K) and two 64x64x64 (dT T^T, T^T W1); hi/lo splits not counted
    "k_bwd_chunk_mma": 2 * (3 * 64 * 128 * 128 + 7 * 64 * 64 * 128 + 2 * 64 * 64 * 64),
}


def measure_backward(args, gdn, torch, np, dev, flush, inp, q, k, v, g, beta, s0):
    """gdn_bwd on the benchmark workload: GPU time per call (caches flushed
    before each), the HBM bytes it must move, and its matrix work; parity of a
    separate call on a token prefix of sequence 0 against the fp64 backward
    oracle."""
    import ctypes
    B, T, h_qk, h_v = inp.B, inp.T, inp.h_qk, inp.h_v
    n_seqs = inp.n_seqs
    r = np.random.default_rng(77)
    f32_io = inp.io_dtype != "bf16"
    d_out = torch.from_numpy(r.standard_normal(inp.v.shape).astype(np.float32)).to(dev, v.dtype)
    d_fin = torch.from_numpy((0.1 * r.standard_normal((n_seqs, h_v, 128, 128))).astype(np.float32)).to(dev)
    cu = None if inp.cu_seqlens is None else [int(x) for x in inp.cu_seqlens]
    desc, keep = gdn.binding.make_desc(B, T, h_qk, h_v, cu_seqlens=cu,
                                       io_dtype=gdn.binding.GDN_F32 if f32_io else gdn.binding.GDN_BF16)
    need = gdn.load_library().gdn_bwd_workspace_bytes(ctypes.byref(desc))
    ws = torch.empty(need, dtype=torch.uint8, device=dev)

    def call():
        return gdn.bwd(q, k, v, g, beta, d_out, scale=inp.scale, initial_state=s0, d_final_state=d_fin,
                       cu_seqlens=cu, workspace=ws)

    for _ in range(2):
        call()
    torch.cuda.synchronize()
    marks = []
    for _ in range(args.bwd_steps):
        flush.zero_()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        call()
        b.record()
        marks.append((a, b))
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in marks]))
    tokens = B * T
    n_chunks = gdn.plan(B, T, h_qk, h_v, cu_seqlens=cu)["n_chunks_total"]
    e_io = 4 if f32_io else 2
    nbytes = tokens * (4 * h_qk * 128 * e_io + 3 * h_v * 128 * e_io + 16 * h_v) + \
        ((s0 is not None) + 2) * n_seqs * h_v * 128 * 128 * 4
    flops = {kname: f * n_chunks * h_v for kname, f in BWD_KERNEL_FLOPS.items()}
    # parity on a prefix: the first 2048 tokens of sequence 0 as a sequence of their own
    n_tok = min(2048, T if inp.cu_seqlens is None else int(inp.cu_seqlens[1]))
    from oracle import gdn_sequential_bwd
    pq, pk, pv = (x[:1, :n_tok].contiguous() for x in (q, k, v))
    pg, pb, pdo = g[:1, :n_tok].contiguous(), beta[:1, :n_tok].contiguous(), d_out[:1, :n_tok].contiguous()
    ps0 = None if s0 is None else s0[:1].contiguous()
    res = gdn.bwd(pq, pk, pv, pg, pb, pdo, scale=inp.scale, initial_state=ps0, d_final_state=d_fin[:1].contiguous())
    torch.cuda.synchronize()
    f64 = lambda x: x[0].float().cpu().numpy().astype(np.float64)  # noqa: E731
    ref = gdn_sequential_bwd(f64(pq), f64(pk), f64(pv), f64(pg), f64(pb), inp.scale, f64(pdo),
                             None if ps0 is None else ps0.cpu().numpy(), d_fin[:1].cpu().numpy())
    par = {}
    for key in ("dq", "dk", "dv", "dg", "dbeta", "d_initial"):
        x = res[key].float().cpu().numpy().astype(np.float64).reshape(ref[key].shape)
        d = np.abs(x - ref[key])
        par[key] = [float(d.max() / np.abs(ref[key]).max()), float(d.sum() / np.abs(ref[key]).sum())]
    print(f"[bench] backward {ms:.3f} ms", file=sys.stderr, flush=True)
    del keep
    return {"ms_per_call": round(ms, 4), "tokens_per_s": round(tokens / (ms * 1e-3), 1),
            "algorithmic_bytes": nbytes, "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 5),
            "gflop_per_kernel": {kname: round(f / 1e9, 2) for kname, f in flops.items()},
            "mfma_peak_tflops": MFMA_PEAK_TFLOPS,
            "precision": ("fp32 q, k, v, dO rounded once to bf16, then " if f32_io else "") +
                         "bf16 MFMA with hi/lo splits of fp32 operands, fp32 accumulation; "
                         "forward re-run as in gdn_fwd",
            "parity_prefix": {"tokens": n_tok, "max_rel_and_mean_rel_l1": par,
                              "tol": ({"all": [1e-2, 5e-3]} if f32_io else
                                      {"dq,dk,dv": [1e-2, 2e-3], "dg,dbeta,d_initial": [1e-3, 1e-4]})}}


def measure_decode(args, gdn, torch, np, dev, flush, timed):
    """One-token decode over args.decode_rows rows at the TP8 head counts
    (h_qk = 2, h_v = 8, bf16 inputs, states drawn N(0, 0.1)): GPU time per
    call (caches flushed before each), HBM roofline, and the outputs of one
    call against the fp64 oracle."""
    from gated_deltanet_chunked_03_amd.synth import make_inputs
    rows, h_qk, h_v = args.decode_rows, 2, 8
    di = make_inputs(name="decode", B=rows, T=1, h_qk=h_qk, h_v=h_v, seed=26, gate="mixed", init_std=0.1)
    dv = lambda a, d=torch.float32: torch.from_numpy(a).to(device=dev, dtype=d)  # noqa: E731
    dq, dk, dvv = dv(di.q, torch.bfloat16), dv(di.k, torch.bfloat16), dv(di.v, torch.bfloat16)
    dg, db, ds = dv(di.g), dv(di.beta), dv(di.initial_state)
    do = torch.empty_like(dvv)
    dso = torch.empty_like(ds)

    def call():
        gdn.decode(dq, dk, dvv, dg, db, ds, scale=di.scale, out=do, state_out=dso)

    for _ in range(20):
        call()
    times = timed(call, max(args.steps, 20))
    us = float(np.mean(times)) * 1e3
    nbytes = decode_bytes(rows, h_qk, h_v)
    gbs = nbytes / (us * 1e-6) / 1e9
    from oracle import gdn_sequential
    qf, kf, vf, gf, bf = di.flat()
    o_ref, s_ref, _ = gdn_sequential(qf, kf, vf, gf, bf, di.scale, di.initial_state, di.flat_cu())
    o_gpu = do.float().cpu().numpy().reshape(o_ref.shape).astype(np.float64)
    s_gpu = dso.cpu().numpy().astype(np.float64)
    err = lambda x, r: (float(np.abs(x - r).max() / np.abs(r).max()),  # noqa: E731
                        float(np.abs(x - r).sum() / np.abs(r).sum()))
    (omx, omean), (smx, smean) = err(o_gpu, o_ref), err(s_gpu, s_ref)
    print(f"[bench] decode {rows} rows: {us:.2f} us/call, {gbs:.0f} GB/s", file=sys.stderr, flush=True)
    traffic = None
    mt = MEASURED_TRAFFIC.get(f"decode{rows}")
    if mt and MEASURED_TRAFFIC["sha256"] == sources_sha256():
        traffic = mt["read"] + mt["write"]
    return {"workload": f"one-token decode: {rows} rows, h_qk={h_qk} h_v={h_v} d_k=d_v=128, bf16 "
                        f"inputs, fp32 states N(0, 0.1), state read and written once per call",
            "kernel": "k_decode", "us_per_call": round(us, 3),
            "tokens_per_s": round(rows / (us * 1e-6), 1),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic, "algorithmic_bytes": nbytes},
            "parity": {"o_max_rel": omx, "o_mean_rel_l1": omean, "state_max_rel": smx,
                       "state_mean_rel_l1": smean}}


class ClockSampler:
    """Samples the GPU shader clock from sysfs (pp_dpm_sclk: the line marked
    '*' holds the current clock) from a host thread, from warm-up to the end
    of the timed steps; summary() reports the samples inside a window."""

    def __init__(self, period_s=0.002):
        import glob
        import threading
        self.paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.period_s, self.samples, self._stop = period_s, [], threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _read(self):
        for path in self.paths:
            try:
                for line in open(path):
                    if "*" in line:
                        return float(line.split(":")[1].strip().lower().split("mhz")[0])
            except (OSError, ValueError, IndexError):
                continue
        return None

    def _run(self):
        while not self._stop.is_set():
            mhz = self._read()
            if mhz is not None:
                self.samples.append((time.time(), mhz))
            self._stop.wait(self.period_s)

    def start(self):
        if self.paths:
            self._thread.start()
        return self

    def stop(self):
        self._stop.set()
        if self.paths:
            self._thread.join()

    def summary(self, t0, t1):
        if not self.paths:
            return {"source": "sysfs pp_dpm_sclk", "samples": 0, "note": "no readable clock file on this host"}
        x = sorted(m for t, m in self.samples if t0 <= t <= t1)
        out = {"source": "sysfs pp_dpm_sclk (current shader clock) read every 2 ms by a host thread",
               "window": "the timed steps (host enqueue start to the final synchronize)", "samples": len(x)}
        if x:
            pick = lambda f: x[min(len(x) - 1, int(f * (len(x) - 1) + 0.5))]  # noqa: E731
            out.update({"min": x[0], "median": pick(0.5), "max": x[-1]})
        return out


def host_info():
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"host_cores_online": os.cpu_count(), "host_cores_available": cores_available(),
            "cpu_model": model}


def cores_available():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # the clocks reach their steady state only after ~100 forwards (about 0.1 s
    # of back-to-back work): fewer warm-up steps time the ramp, not the kernels
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--config", default="tp8",
                    choices=["tiny", "tp8", "tp4", "tp2", "tp1", "tp1_b4", "long"])
    ap.add_argument("--cp-mode", default="auto", choices=["auto", "off", "exact", "warmup"])
    ap.add_argument("--lam", type=float, default=0.0)
    ap.add_argument("--dv-split", type=int, default=0, choices=[0, 1, 2, 4],
                    help="column blocks of d_v in the forward (0 = the planner decides)")
    ap.add_argument("--cpu-tokens", type=int, default=32768,
                    help="tokens of sequence 0 the CPU oracle runs (0 = skip)")
    ap.add_argument("--no-flush", action="store_true", help="skip the cache flush between steps")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step replayed from a HIP graph (reported, not the headline: "
                         "on this stack the replay measured slower than eager launches)")
    ap.add_argument("--bwd-steps", type=int, default=5,
                    help="timed calls of the backward pass on the same workload (0 = skip)")
    ap.add_argument("--decode-rows", type=int, default=256,
                    help="rows (sequences) of the one-token decode measurement at the TP8 head "
                         "counts (0 = skip)")
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="untimed forwards (each after the cache flush, as a step) for this long before "
                         "the warm-up steps, so that the shader clock has left its idle level")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="before warm-up, copy a buffer of this many MiB once (a kernel of known "
                         "traffic that scales the HBM byte counters of a profiled run)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU (the library has no multi-GPU path); use --gpus 1"}))
        sys.exit(2)

    import numpy as np
    import torch

    import gated_deltanet_chunked_03_amd as gdn
    from gated_deltanet_chunked_03_amd.synth import CONFIGS, config_inputs

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    t_gen = time.time()
    inp = config_inputs(args.config)
    print(f"[bench] generated {args.config} in {time.time() - t_gen:.1f}s", file=sys.stderr, flush=True)
    dt = torch.bfloat16 if inp.io_dtype == "bf16" else torch.float32
    dv = lambda a, d=torch.float32: torch.from_numpy(a).to(device=dev, dtype=d)  # noqa: E731
    q, k, v = dv(inp.q, dt), dv(inp.k, dt), dv(inp.v, dt)
    g, beta = dv(inp.g), dv(inp.beta)
    s0 = None if inp.initial_state is None else dv(inp.initial_state)
    B, T, h_qk, h_v = inp.B, inp.T, inp.h_qk, inp.h_v
    n_seqs = inp.n_seqs
    out = torch.empty_like(v)
    fs = torch.empty((n_seqs, h_v, 128, 128), dtype=torch.float32, device=dev)
    pl = gdn.plan(B, T, h_qk, h_v, io_dtype=0 if inp.io_dtype == "bf16" else 1,
                  cp_mode=args.cp_mode, lam=args.lam, dv_split=args.dv_split)
    ws = torch.empty(max(pl["workspace_bytes"], 256), dtype=torch.uint8, device=dev)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)

    if args.copy_mib > 0:
        src = torch.ones(args.copy_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def step():
        gdn.fwd(q, k, v, g, beta, scale=inp.scale, initial_state=s0, cp_mode=args.cp_mode,
                lam=args.lam, workspace=ws, out=out, final_state=fs, dv_split=args.dv_split)

    clock = ClockSampler().start()
    # The power controller raises the shader clock over tens of milliseconds of
    # load after the idle input setup; the forwards below (each after the flush,
    # exactly as a step) let it settle, so that the warm-up and timed steps
    # measure the kernels rather than the ramp. Reported as "settle".
    settle_steps, t_settle = 0, time.time()
    while (time.time() - t_settle) * 1e3 < args.settle_ms:
        if not args.no_flush:
            flush.zero_()
        step()
        settle_steps += 1
        if settle_steps % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    settle = {"ms": round((time.time() - t_settle) * 1e3, 1), "forwards": settle_steps}
    for _ in range(args.warmup):
        if not args.no_flush:
            flush.zero_()
        step()
    torch.cuda.synchronize()
    print(f"[bench] warmup done, plan L={pl['L']} segments={pl['n_segments']}",
          file=sys.stderr, flush=True)

    def timed(run, n):
        """GPU ms of n steps: HIP events on the stream around each step (the
        cache flush before it stays outside the interval); one sync at the end,
        so the host enqueues ahead of the GPU."""
        marks = []
        for _ in range(n):
            if not args.no_flush:
                flush.zero_()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            run()
            b.record()
            marks.append((a, b))
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in marks]

    # eager launches: the four kernels back to back on the stream
    torch.cuda.synchronize()
    t0 = time.time()
    eager_ms = timed(step, args.steps)
    wall = time.time() - t0
    clock_timed = clock.summary(t0, t0 + wall)

    # the same four launches replayed from a HIP graph (no host launch gaps);
    # every replay is checked against the eager result before it is timed
    graph_ms, graph_ok = None, False
    if args.graph:
        step()
        torch.cuda.synchronize()
        o_ref, s_ref = out.clone(), fs.clone()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        graph_ok = True
        for _ in range(3):
            out.zero_()
            graph.replay()
            torch.cuda.synchronize()
            graph_ok &= bool(torch.equal(out, o_ref)) and bool(torch.equal(fs, s_ref))
            step()   # eager work between replays
            torch.cuda.synchronize()
        if graph_ok:
            graph_ms = timed(graph.replay, args.steps)
        print(f"[bench] graph replays {'match' if graph_ok else 'DIFFER from'} the eager result",
              file=sys.stderr, flush=True)

    # per-kernel times (events between the kernels; eager, cold caches)
    t_pk = time.time()
    gdn.profile_enable(True)
    per = {"prep": [], "cp_prep": [], "cp_combine": [], "fwd": [], "total": []}
    for _ in range(args.steps):
        if not args.no_flush:
            flush.zero_()
        step()
        for key, val in gdn.profile_read().items():
            per[key].append(val)
    # warm-cache figure (no flush), for reference
    warm = []
    for _ in range(max(3, args.steps // 2)):
        step()
        warm.append(gdn.profile_read()["total"])
    gdn.profile_enable(False)
    clock.stop()
    clock_pk = clock.summary(t_pk, time.time())
    clock_pk["window"] = "the per-kernel pass (one synchronisation per step)"
    clock_timed["note"] = ("the power controller's averaged clock: it includes the gaps between "
                           "steps and the cache flushes, not only the kernels")
    print(f"[bench] timed {args.steps} steps in {wall:.2f}s", file=sys.stderr, flush=True)

    backward = None
    if args.bwd_steps > 0:
        backward = measure_backward(args, gdn, torch, np, dev, flush, inp, q, k, v, g, beta, s0)

    decode = None
    if args.decode_rows > 0:
        decode = measure_decode(args, gdn, torch, np, dev, flush, timed)

    mean = {key: float(np.mean(vals)) for key, vals in per.items()}
    eager = float(np.mean(eager_ms))
    ms = eager
    tokens = B * T
    value = tokens / (ms * 1e-3)
    nbytes = algorithmic_bytes(B, T, h_qk, h_v, e_io=2 if inp.io_dtype == "bf16" else 4,
                               initial=s0 is not None, final=True, n_seqs=n_seqs)
    flops = algorithmic_flops(B, T, h_qk, h_v)
    step_gbs = nbytes / (ms * 1e-3) / 1e9
    k_s = mean[DOMINANT_KERNEL] * 1e-3
    k_gbs = nbytes / k_s / 1e9
    # counter traffic (valid for the sources it was taken on, the default plan only)
    mt = MEASURED_TRAFFIC.get(args.config) if MEASURED_TRAFFIC["sha256"] == sources_sha256() else None
    if args.cp_mode != "auto" or args.lam != 0.0:
        mt = None
    step_traffic = round(sum(r + w for r, w in mt["per_kernel"].values())) if mt else None
    kernel_traffic = round(sum(mt["per_kernel"][mt["dominant"]])) if mt else None
    roofline = {"bound": "hbm", "scope": "whole forward step (ms_per_step)",
                "achieved": round(step_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(step_gbs / HBM_PEAK_GBS, 4), "traffic": step_traffic,
                "algorithmic_bytes": nbytes,
                "kernel": {"name": "k_fwd_ws" if inp.io_dtype == "bf16" else "k_fwd16<float>",
                           "ms": round(mean[DOMINANT_KERNEL], 4),
                           "achieved": round(k_gbs, 1), "frac": round(k_gbs / HBM_PEAK_GBS, 4),
                           "traffic": kernel_traffic,
                           "note": "the step's algorithmic bytes over this kernel's event-timed "
                                   "duration alone"},
                "traffic_per_kernel_mb": ({kname: [round(r / 1e6, 1), round(w / 1e6, 1)]
                                           for kname, (r, w) in mt["per_kernel"].items()} if mt else None)}
    mfma = {"algorithmic_gflop": round(flops / 1e9, 2),
            "achieved_tflops_step": round(flops / (ms * 1e-3) / 1e12, 2),
            "peak_tflops": MFMA_PEAK_TFLOPS,
            "frac_step": round(flops / (ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS, 4),
            "frac_dominant_kernel": round(flops / k_s / 1e12 / MFMA_PEAK_TFLOPS, 4),
            # matrix work the step's kernels execute (rocprofv3 MfmaFlopsF16 + MfmaFlopsBF16)
            "executed_gflop_step_measured": round(mt["mfma_flops"] / 1e9, 2) if mt else None,
            "frac_executed_step": (round(mt["mfma_flops"] / (ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS, 4)
                                   if mt else None)}

    cpu = None
    parity = None
    boundary = None
    if args.cpu_tokens > 0:
        from oracle import gdn_sequential
        n_tok = min(args.cpu_tokens, T if inp.cu_seqlens is None else int(inp.cu_seqlens[1]))
        threads = max(1, min(cores_available(), 16, h_v))
        qf, kf, vf, gf, bf = (a[:n_tok] for a in inp.flat())
        s0_np = None if inp.initial_state is None else inp.initial_state[:1]
        # the oracle also keeps its states at the segment boundaries inside the prefix
        stride = 64 * pl["L"] if pl["cp_on"] else 0
        n_snap = (n_tok // stride + 1) if stride else 0
        runs, t1 = 0, time.time()
        while runs == 0 or time.time() - t1 < 3.0:   # repeat to a few seconds of wall time
            o_ref, _, snaps = gdn_sequential(qf, kf, vf, gf, bf, inp.scale, s0_np, None,
                                             snap_stride=stride, n_snap=n_snap, n_threads=threads)
            runs += 1
        cpu_s = (time.time() - t1) / runs
        cpu = {"value": round(n_tok / cpu_s, 1), "unit": "tokens/s", "cores": threads,
               "kind": "oracle",
               "sample": f"first {n_tok} tokens of sequence 0, all {h_v} value heads, fp64 "
                         f"token-by-token recurrence, one thread per head; mean of {runs} runs, "
                         f"{cpu_s:.2f}s each",
               **host_info()}
        o_gpu = out[0, :n_tok].float().cpu().numpy().astype(np.float64)
        d = np.abs(o_gpu - o_ref)
        parity = {"tokens": n_tok, "max_rel": float(d.max() / np.abs(o_ref).max()),
                  "mean_rel_l1": float(d.sum() / np.abs(o_ref).sum()),
                  "tol_max_rel": 1e-2, "tol_mean_rel": 2e-3}
        if stride and n_snap > 1:
            # the segment initial states the forward used (one debug call, same plan)
            _, _, dbg = gdn.fwd(q, k, v, g, beta, scale=inp.scale, initial_state=s0, cp_mode=args.cp_mode,
                                lam=args.lam, workspace=ws, debug=True, dv_split=args.dv_split)
            seg = dbg["seg_state"].cpu().numpy()
            path = dbg["path"].cpu().numpy()[0]
            P0 = min(pl["P_max"], n_snap)
            per_head = []
            for h in range(h_v):
                rel = [float(np.linalg.norm(seg[s, h] - snaps[0, h, s]) / np.linalg.norm(snaps[0, h, s]))
                       for s in range(1, P0) if 64 * pl["L"] * s < n_tok]
                per_head.append(round(max(rel), 7) if rel else None)
            codes = {0: "exact", 1: "warm-up", 2: "mixed", 3: "start only", -1: "not split"}
            boundary = {"metric": "max over boundaries of |S0 - S_ref|_F / |S_ref|_F",
                        "tol": 1e-3, "boundaries": P0 - 1,
                        "per_head": per_head,
                        "path_per_head": [codes.get(int(c), str(int(c))) for c in path],
                        "head_class": list(inp.head_class),
                        "max_warmup_heads": max([e for e, c in zip(per_head, path) if c == 1 and e is not None],
                                                default=None),
                        "max_exact_heads": max([e for e, c in zip(per_head, path) if c != 1 and e is not None],
                                               default=None)}

    cfg = CONFIGS[args.config]
    workload = (f"{args.config}: B={B} T={T} h_qk={h_qk} h_v={h_v} d_k=d_v=128 chunk=64 "
                f"{inp.io_dtype} inputs, fp32 state, heads {','.join(inp.head_class)}")
    qs = lambda f: float(np.percentile(eager_ms, f))  # noqa: E731
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "settle": settle, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak",
        "vs_baseline": (round(value / (T / (PAGES_MS[args.config] * 1e-3)), 3)
                        if args.config in PAGES_MS and B == 1 else None),
        "baseline": ({"value": round(T / (PAGES_MS[args.config] * 1e-3), 1), "unit": "tokens/s",
                      "source": "the pages' FlashQLA forward time for this shape on an H200 (context)",
                      "ms": PAGES_MS[args.config]} if args.config in PAGES_MS else None),
        "dtype": inp.io_dtype, "data": "synthetic",
        "config": {"workload": workload, "B": B, "T": T, "h_qk": h_qk, "h_v": h_v, "d": 128,
                   "chunk": 64, "cp_mode": args.cp_mode, "dv_split": pl["dv_split"], "seed": cfg["seed"]},
        "roofline": roofline, "cpu_baseline": cpu,
        "step_ms_stats": {"median": round(qs(50), 4), "p10": round(qs(10), 4), "p90": round(qs(90), 4),
                          "min": round(min(eager_ms), 4), "max": round(max(eager_ms), 4)},
        "gpu_clock_mhz": clock_timed, "gpu_clock_mhz_per_kernel_pass": clock_pk,
        "launch": "eager",
        "eager_ms_per_step": round(eager, 4),
        "graph_ms_per_step": round(float(np.mean(graph_ms)), 4) if graph_ok else None,
        "kernels_ms": {key: round(val, 4) for key, val in mean.items()},
        "warm_cache_ms_per_step": round(float(np.mean(warm)), 4),
        "mfma": mfma, "parity": parity, "boundary_state_error": boundary,
        "backward": backward, "decode": decode,
        "plan": {key: pl[key] for key in ("L", "n_segments", "P_max", "cp_on", "dv_split", "cp_layout",
                                          "warmup_chunks", "n_cu", "lambda")},
        "precision": ("fp16 matrix-core operands for the chunk chain (state, V', K, Q, "
                      "T diag(beta), P), V through an exact bf16 identity product, fp32 "
                      "accumulation and fp32 state" if inp.io_dtype == "bf16" else
                      "fp16 matrix-core operands from fp32 inputs, fp32 accumulation and state"),
        "wall_s": round(wall, 3),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
