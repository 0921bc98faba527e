"""Builds the gfx950 HIP library (libmoe_gfx950.so) in-tree with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmoe_gfx950.so")
SOURCES = ["moe_api.cpp", "moe_static.hip", "prof.cpp", "route.hip", "union.hip", "ffn_gemv.hip",
           "ffn_gemv_i3.hip", "ffn_gemv_f4.hip", "ffn_mfma.hip", "combine.hip", "glue.hip", "probe.hip",
           "tier.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-function",
    # no packed-fp32 VALU instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    return subprocess.run(cmd, capture_output=True, text=True)


def build(verbose: bool = False, jobs: int | None = None, extra: list | None = None,
          out: str | None = None) -> str:
    """Each source compiled to an object in parallel (jobs, default: up to 8), then linked
    into `out` (default: the in-tree library); `extra`: more hipcc flags for every step."""
    jobs = jobs or max(1, min(8, os.cpu_count() or 1))
    extra = list(extra or [])
    lib = out or LIB
    objdir = tempfile.mkdtemp(prefix="moe_build_")
    try:
        objs = [os.path.join(objdir, s + ".o") for s in SOURCES]
        cmds = [[HIPCC] + FLAGS + extra + ["-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
        with ThreadPoolExecutor(max_workers=jobs) as ex:
            results = list(ex.map(lambda c: _run(c, verbose), cmds))
        for s, res in zip(SOURCES, results):
            if res.returncode != 0:
                sys.stderr.write(res.stdout + res.stderr)
                raise RuntimeError(f"hipcc failed compiling {s}")
        tmp = lib + ".tmp"
        res = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + extra + objs + ["-o", tmp], verbose)
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            raise RuntimeError(f"hipcc failed linking {os.path.basename(lib)}")
        os.replace(tmp, lib)
    finally:
        shutil.rmtree(objdir, ignore_errors=True)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
