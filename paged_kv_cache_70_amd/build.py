"""Build ``libpaged_kv.so`` (the C-ABI library) in-tree with hipcc for gfx950,
and beside it ``libpaged_kv_timeline.so``: the same library with the
persistent decode kernel built with -DPA_TIMELINE (per-wavefront and per-unit
timestamps, read by ``paged_kv_cache_70_amd.timeline``; not used otherwise).

Usage: ``python -m paged_kv_cache_70_amd.build`` (or ``build()`` from Python).
Every call recompiles.  Sources are compiled in parallel, then linked.
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
LIB = os.path.join(PKG, "libpaged_kv.so")
TIMELINE_LIB = os.path.join(PKG, "libpaged_kv_timeline.so")
TIMELINE_SOURCE = "pa_decode_mfma.hip"
SOURCES = ["pa_api.hip", "pa_write.hip", "pa_decode.hip", "pa_decode_mfma.hip", "pa_prefill.hip", "pa_measure.hip",
           "pa_check.hip"]
HOST_SOURCES = ["pa_block_manager.cpp"]      # host-only C++ (no device code)
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall"]
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from forming v_pk_{add,mul,fma}_f32.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature: drop that warning
    noise = "'-packed-fp32-ops' is not a recognized feature for this target"
    err = "\n".join(x for x in r.stderr.splitlines() if noise not in x)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    return err


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    inc = os.path.join(ROOT, "include")

    def compile_one(src, defines=()):
        obj = os.path.join(objdir, src.replace(".hip", "_timeline.o" if defines else ".o"))
        cmd = [hipcc, *HIP_FLAGS, *defines, "-I", inc, "-c", os.path.join(CSRC, src), "-o", obj]
        err = _run(cmd)
        if verbose and err.strip():
            print(err, file=sys.stderr)
        return obj

    def compile_host(src):
        obj = os.path.join(objdir, src.replace(".cpp", ".o"))
        cxx = shutil.which("g++") or shutil.which("c++")
        if not cxx:
            raise RuntimeError("no host C++ compiler (g++) found")
        err = _run([cxx, *HOST_FLAGS, "-I", inc, "-c", os.path.join(CSRC, src), "-o", obj])
        if verbose and err.strip():
            print(err, file=sys.stderr)
        return obj

    with cf.ThreadPoolExecutor(max_workers=len(SOURCES) + len(HOST_SOURCES) + 1) as ex:
        futs = [ex.submit(compile_one, s) for s in SOURCES] + [ex.submit(compile_host, s) for s in HOST_SOURCES]
        tl_fut = ex.submit(compile_one, TIMELINE_SOURCE, ("-DPA_TIMELINE",))
        objs = [f.result() for f in futs]
        tl_obj = tl_fut.result()
    for out, parts in ((LIB, objs),
                       (TIMELINE_LIB, [tl_obj if os.path.basename(o) == TIMELINE_SOURCE.replace(".hip", ".o") else o
                                       for o in objs])):
        tmp = out + ".tmp"
        _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *parts])
        os.replace(tmp, out)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
