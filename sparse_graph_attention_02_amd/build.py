"""Build libgraph_attn.so in-tree with hipcc for gfx950.

    python -m sparse_graph_attention_02_amd.build [-v]

Every call recompiles every source (a few seconds per file, files in parallel).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libgraph_attn.so")
ARCH = os.environ.get("GA_OFFLOAD_ARCH", "gfx950")

SOURCES = ["plan.cpp", "api.cpp", "fwd.hip", "bwd.hip", "bwd_gat.hip", "bwd_gatv2.hip",
           "reduce.hip", "probe.hip", "noalloc.hip"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]
# device code: gfx950 only; packed fp32 ops are disabled for all device code
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
          "-packed-fp32-ops"]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _rocm_include() -> str:
    return os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "include")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    path = os.path.join(CSRC, src)
    if src.endswith(".hip"):
        cmd = [_hipcc(), "-x", "hip", *COMMON, *DEVICE, "-c", path, "-o", obj]
    else:  # host-only C++ (still through hipcc for the HIP runtime headers)
        cmd = [_hipcc(), "-x", "c++", "-D__HIP_PLATFORM_AMD__=1", "-I", _rocm_include(), *COMMON,
               "-c", path, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, flush=True)
    return obj


def build(verbose: bool = False, out: str | None = None, defines=()) -> str:
    """Compile and link; ``out`` and ``defines`` (e.g. ["GA_UNROLL=8"]) build a variant
    library elsewhere (tuning); the default is the in-tree libgraph_attn.so."""
    global OBJ
    lib = out or LIB
    obj_dir = OBJ if out is None else os.path.splitext(out)[0] + "_obj"
    os.makedirs(obj_dir, exist_ok=True)
    saved = OBJ, list(COMMON)
    OBJ = obj_dir
    COMMON.extend(f"-D{d}" for d in defines)
    try:
        return _build(verbose, lib)
    finally:
        OBJ = saved[0]
        COMMON[:] = saved[1]


def _build(verbose: bool, lib: str) -> str:
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = lib + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
