"""Build libkvq.so in-tree for gfx950 with hipcc.

Each translation unit is compiled to an object in parallel, then linked into
``kv_cache_int4_amd/libkvq.so``.  Run as ``python -m kv_cache_int4_amd.build``.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libkvq.so")

SOURCES = ["kvq_api.cpp", "kvq_codec.hip", "kvq_mixed.hip", "kvq_attn.hip", "kvq_attn_f16.hip", "kvq_noalloc.hip",
           "kvq_diag.hip"]

# Per-source flags.  Attention: matrix instructions write their results to
# VGPRs even where the kernel also uses AGPRs (its D=256 form needs more
# than 256 registers): the compiler then keeps the blocks in flight, not
# the score accumulators, in the AGPRs, and no longer copies every score
# out of them (about a fifth fewer VALU instructions per D=256 block).
PER_SOURCE = {"kvq_attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}

ARCH = "gfx950"
COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    f"--offload-arch={ARCH}",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libkvq")


def _compile(src: str, extra: list[str]) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMMON, *PER_SOURCE.get(src, []), *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    """Compile every source for gfx950 and link libkvq.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    extra = list(extra or [])
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
