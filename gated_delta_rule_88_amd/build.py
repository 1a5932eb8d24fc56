"""Build libgdr.so (the C-ABI library) for gfx950 with hipcc, in-tree.

Every source is compiled to an object in its own hipcc process (in
parallel), then the objects are linked into gated_delta_rule_88_amd/libgdr.so.
Each translation unit holds its kernels and their launchers, so no
relocatable device code is needed.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libgdr.so")
OBJ = os.path.join(ROOT, "_build")
SOURCES = ["gdr_api.hip", "gdr_decode.hip", "gdr_fwd.hip", "gdr_wy.hip", "gdr_scan.hip", "gdr_segment.hip",
           "gdr_bwd.hip", "gdr_bwd_chain.hip",
           "gdr_noalloc.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 VALU forms are switched off for every device pass; the host
# pass does not know the feature and says so, which is harmless.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-fvisibility=hidden", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include")]
NOISE = "'-packed-fp32-ops' is not a recognized feature"


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(ln for ln in res.stderr.splitlines() if NOISE not in ln)
    return res.returncode, err


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every HIP source and link gated_delta_rule_88_amd/libgdr.so."""
    os.makedirs(OBJ, exist_ok=True)
    objs = [os.path.join(OBJ, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    cmds = [[HIPCC, *FLAGS, "-c", "-o", o, os.path.join(CSRC, s)] for s, o in zip(SOURCES, objs)]
    with ThreadPoolExecutor(max_workers=max(1, min(jobs, len(cmds)))) as ex:
        results = list(ex.map(_run, cmds))
    for (rc, err), s in zip(results, SOURCES):
        if rc != 0:
            raise RuntimeError(f"hipcc failed on {s} ({rc}):\n{err}")
        if verbose and err.strip():
            print(err, file=sys.stderr)
    tmp = LIB + ".tmp"
    rc, err = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs])
    if rc != 0:
        raise RuntimeError(f"link failed ({rc}):\n{err}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
