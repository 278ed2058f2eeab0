"""Build the HIP library ``_build/libgdn.so`` in-tree with hipcc for gfx950,
and beside it ``_build/libgdn_poison.so``: the same sources with LDS poisoning
(every kernel first fills its shared memory with NaN words; a debug build that
the GPU tests compare with the normal one).

    python -m gated_deltanet_chunked_03_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(BUILD, "libgdn.so")
LIB_POISON = os.path.join(BUILD, "libgdn_poison.so")
SOURCES = [os.path.join(CSRC, "gdn_kernels.hip"), os.path.join(CSRC, "gdn_fwd16.hip"),
           os.path.join(CSRC, "gdn_bwd.hip"), os.path.join(CSRC, "gdn_noalloc.hip"),
           os.path.join(CSRC, "gdn_api.cpp")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # the memory-clause scheduler keeps each wave's loads and LDS reads grouped
    # ahead of their uses (measured: the chain kernels' best)
    "-mllvm", "-amdgpu-sched-strategy=max-memory-clause",
    # packed fp32 ops are kept out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _compile(target: str, extra: list, verbose: bool) -> None:
    tmp = target + f".tmp{os.getpid()}"
    cmd = [HIPCC, *FLAGS, *extra, *SOURCES, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, file=sys.stderr)
    os.replace(tmp, target)


def build(verbose: bool = False, poison: bool = True) -> str:
    """Compile every source into the in-tree shared library (always recompiles),
    and the LDS-poisoning debug build beside it (poison=True)."""
    from concurrent.futures import ThreadPoolExecutor
    os.makedirs(BUILD, exist_ok=True)
    jobs = [(LIB, [])] + ([(LIB_POISON, ["-DGDN_LDS_POISON"])] if poison else [])
    with ThreadPoolExecutor(len(jobs)) as ex:
        for f in [ex.submit(_compile, t, e, verbose) for t, e in jobs]:
            f.result()
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
