"""Full-size workloads on the GPU against the fp64 oracle, every output element.

Each case runs the forward exactly as bench.py does (AUTO context parallelism,
256 CUs), compares o and the final state with the oracle at the stated
tolerance, and checks each segment's initial state against the oracle's state
at that boundary: exact boundaries to fp32 accuracy, warm-up boundaries within
1e-3 relative (Frobenius) of the true state.
"""
from __future__ import annotations

import numpy as np
import pytest

from gated_deltanet_chunked_03_amd.synth import config_inputs
from gpu_util import BOUNDARY_TOL, STATE_MAX_TOL, STATE_MEAN_TOL, assert_within_tolerance, oracle_run, to_device

pytestmark = pytest.mark.gpu

CASES = [("tiny", "auto"), ("tp8", "auto"), ("tp4", "auto"), ("tp2", "auto"), ("tp1", "auto"),
         ("tp1_b4", "auto"), ("tp1_b4", "off"), ("long", "auto")]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,mode", CASES, ids=[f"{n}-{m}" for n, m in CASES])
def test_workload_parity(name, mode):
    import torch
    import gated_deltanet_chunked_03_amd as gdn

    inp = config_inputs(name)
    print(f"\n[{name}/{mode}] B={inp.B} T={inp.T} heads {inp.h_qk}/{inp.h_v} {inp.io_dtype}", flush=True)
    d = to_device(inp)
    o, S, info = gdn.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], scale=inp.scale,
                         initial_state=d["initial_state"], cp_mode=mode, debug=True)
    torch.cuda.synchronize()
    plan = info["plan"]
    L = plan["L"]
    print(f"  plan L={L} P={plan['P_max']} segments={plan['n_segments']} cp_on={plan['cp_on']}",
          flush=True)
    seg = info["seg_state"].cpu().numpy()
    path = info["path"].cpu().numpy()
    o_gpu = o.float().cpu().numpy().reshape(inp.B * inp.T, inp.h_v, -1)
    S_gpu = S.cpu().numpy()
    del o, S, d, info
    torch.cuda.empty_cache()

    P = plan["P_max"]
    o_ref, S_ref, snaps = oracle_run(inp, snap_stride=64 * L if P > 1 else 0, n_snap=P)
    mx, mean = assert_within_tolerance(o_gpu, o_ref)
    smx, smean = assert_within_tolerance(S_gpu, S_ref, "final_state", STATE_MAX_TOL, STATE_MEAN_TOL)
    print(f"  o: max-rel {mx:.3e} mean-rel {mean:.3e}; final state {smx:.2e}/{smean:.2e}", flush=True)

    if P > 1:
        for n in range(inp.n_seqs):
            for h in range(inp.h_v):
                rel = [np.linalg.norm(seg[n * P + s, h] - snaps[n, h, s]) /
                       np.linalg.norm(snaps[n, h, s]) for s in range(1, P)]
                kind = {1: "warm-up", 0: "exact", 2: "mixed", 3: "start", -1: "whole"}[int(path[n, h])]
                if n == 0:
                    print(f"  head {h} ({inp.head_class[h]}, {kind}): max boundary state error {max(rel):.2e}")
                assert max(rel) <= BOUNDARY_TOL, (n, h, kind)
                if kind == "exact":
                    assert max(rel) <= BOUNDARY_TOL, (n, h)
                if inp.head_class[h] == "fast":
                    assert kind == "warm-up"
                elif inp.head_class[h] in ("slow", "near1"):
                    assert kind == "exact"
