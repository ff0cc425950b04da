"""Build ``libpagedkv.so`` in-tree: HIP sources with hipcc for gfx950, the host pool with g++.

Run ``python -m paged_kv_cache_127_amd.build`` (or ``__graft_entry__.build()``). Objects go to
``_build/`` at the repository root; the shared library lands next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpagedkv.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
    # no packed fp32 instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]
CXX_FLAGS = ["-O2", "-fPIC", "-std=c++17", "-Wall", "-I", INCLUDE]

HIP_SOURCES = ["api.hip", "decode_mfma.hip", "decode_valu.hip", "splitk_reduce.hip",
               "append_cow.hip", "swap.hip", "row_states.hip", "probe.hip"]
CXX_SOURCES = ["pool.cpp", "prefix_index.cpp"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "is not a recognized feature for this target" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, jobs: int = 8, out: str = LIB, defines=(),
          build_dir: str = BUILD) -> str:
    os.makedirs(build_dir, exist_ok=True)
    jobs_list = []
    dflags = [f"-D{d}" for d in defines]
    for src in HIP_SOURCES:
        obj = os.path.join(build_dir, src + ".o")
        jobs_list.append([HIPCC, *HIP_FLAGS, *dflags, "-c", os.path.join(CSRC, src), "-o", obj])
    cxx = shutil.which("g++") or "g++"
    for src in CXX_SOURCES:
        obj = os.path.join(build_dir, src + ".o")
        jobs_list.append([cxx, *CXX_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        outs = list(ex.map(_run, jobs_list))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    objs = [c[c.index("-o") + 1] for c in jobs_list]
    tmp = out + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
