"""gdn_fwd_noalloc (the allocation-free forward, include/gdn.h) against gdn_fwd
on the GPU: two calls in a row, the second smaller, each compared element by
element with gdn_fwd on the same inputs; a descriptor above the scratch size
is refused before any launch."""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from gated_deltanet_chunked_03_amd import binding as B
from gated_deltanet_chunked_03_amd.synth import make_inputs

pytestmark = pytest.mark.gpu


def _on_gpu(inp):
    dev = torch.device("cuda", 0)
    t = lambda a, d=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to(device=dev, dtype=d)
    return (t(inp.q, torch.bfloat16), t(inp.k, torch.bfloat16), t(inp.v, torch.bfloat16), t(inp.g), t(inp.beta))


@pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")
def test_noalloc_matches_fwd_two_calls():
    # the first call splits its sequence (AutoCP on: maps, segment states and
    # flags live in the scratch array); the second is smaller and reuses the
    # array's stale contents
    for seed, T, h_qk, h_v in [(11, 8192, 2, 8), (12, 1000, 1, 2)]:
        print(f"noalloc case seed={seed} T={T} h_qk={h_qk} h_v={h_v}", flush=True)
        inp = make_inputs(B=1, T=T, h_qk=h_qk, h_v=h_v, seed=seed)
        q, k, v, g, beta = _on_gpu(inp)
        plan = B.plan(1, T, h_qk, h_v, n_cu=0)
        assert plan["workspace_bytes"] <= B.NOALLOC_SCRATCH_BYTES
        o_ref, s_ref = B.fwd(q, k, v, g, beta, scale=inp.scale)
        o_na, s_na = B.fwd_noalloc(q, k, v, g, beta, scale=inp.scale)
        torch.cuda.synchronize()
        # the same kernels on the same inputs: equal to the last bit
        assert torch.equal(o_na, o_ref)
        assert torch.equal(s_na, s_ref)
        if seed == 11:
            assert plan["cp_on"] == 1


@pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")
def test_noalloc_refuses_oversized_descriptor():
    lib = B.load_library()
    desc, keep = B.make_desc(16, 65536, 16, 64)
    need = lib.gdn_fwd_workspace_bytes(ctypes.byref(desc))
    assert need > B.NOALLOC_SCRATCH_BYTES
    nul = ctypes.c_void_p(0x1000)   # never dereferenced: the size check comes first
    st = lib.gdn_fwd_noalloc(ctypes.byref(desc), nul, nul, nul, nul, nul, 0.1, None, None, nul, None, None)
    assert st == 7, B.STATUS_NAMES[st]   # GDN_ERR_WORKSPACE_TOO_SMALL
    assert b"scratch" in lib.gdn_last_error()
    del keep
