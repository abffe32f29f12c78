"""Builds libdflash.so for gfx950 in-tree with hipcc (one shared library, C ABI).

Each HIP source is compiled in parallel into _build/, then linked; the library lands next to
this file, where the binding loads it."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libdflash.so")
SOURCES = ["dflash.hip", "gemm.hip", "gemm_tile.hip", "rows.hip", "attention.hip", "select.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMPILE_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU ops are kept out of the generated code on purpose
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature; that is harmless
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in l]
    return res.returncode, "\n".join(msgs)


def build(verbose: bool = False) -> str:
    """Compiles every HIP source and links libdflash.so (always rebuilds).  Returns the path."""
    os.makedirs(OBJ, exist_ok=True)
    jobs = []
    for s in SOURCES:
        obj = os.path.join(OBJ, s.replace(".hip", ".o"))
        jobs.append((obj, [HIPCC, *COMPILE_FLAGS, "-c", os.path.join(CSRC, s), "-o", obj]))
    with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 4, 8)) as ex:
        results = list(ex.map(lambda j: _run(j[1]), jobs))
    for (obj, cmd), (rc, msg) in zip(jobs, results):
        if verbose:
            print(" ".join(cmd), flush=True)
        if rc != 0:
            raise RuntimeError(f"hipcc failed on {os.path.basename(obj)}:\n{msg}")
        if verbose and msg:
            print(msg, file=sys.stderr)
    tmp = LIB + ".tmp"
    rc, msg = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *[o for o, _ in jobs], "-o", tmp])
    if rc != 0:
        raise RuntimeError("link failed:\n" + msg)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
