"""Build libpkv.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Every source is compiled to an object in parallel, then linked in-tree into
``paged_kv_cache_scatter_amd/libpkv.so``; the benchmark's read-bandwidth
probes go into ``libpkv_probe.so`` beside it, and a copy of the library whose
decode kernel records phase timestamps into ``libpkv_trace.so``. Run as ``python -m
paged_kv_cache_scatter_amd.build``.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libpkv.so")
SOURCES = ["pkv_api.hip", "pkv_write.hip", "pkv_decode.hip", "pkv_prefill.hip"]
HOST_SOURCES = ["pkv_sched.cpp"]   # host-only C++ (the scheduler above the kernels)
# read-bandwidth probes for the benchmark, in a library of their own
PROBE_SOURCE = "pkv_probe.hip"
PROBE_LIB = os.path.join(PKG, "libpkv_probe.so")
# the same library with the decode kernel's phase timestamps compiled in
# (PKV_PHASE_TRACE), for the benchmark's --phase-trace
TRACE_LIB = os.path.join(PKG, "libpkv_trace.so")
ARCH = "gfx950"

# Packed-fp32 VALU ops are switched off for the device code; hipcc's host pass
# does not know the feature and says so, which is harmless.
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libpkv.so)")


def cxx() -> str:
    for cand in (os.environ.get("CXX"), shutil.which("g++"), shutil.which("c++")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("no host C++ compiler (g++) found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(line for line in r.stderr.splitlines()
                    if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = False) -> str:
    cc = hipcc()
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, s.replace(".hip", ".o")) for s in SOURCES]
    cmds = [[cc, *FLAGS, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
    for s in HOST_SOURCES:
        o = os.path.join(objdir, s.replace(".cpp", ".o"))
        cmds.append([cxx(), "-O2", "-std=c++17", "-fPIC", "-Wall", "-c", os.path.join(CSRC, s),
                     "-o", o])
        objs.append(o)
    probe_tmp = PROBE_LIB + ".tmp"
    cmds.append([cc, *FLAGS, "-shared", os.path.join(CSRC, PROBE_SOURCE), "-o", probe_tmp])
    trace_obj = os.path.join(objdir, "pkv_decode_trace.o")
    cmds.append([cc, *FLAGS, "-DPKV_PHASE_TRACE", "-c", os.path.join(CSRC, "pkv_decode.hip"),
                 "-o", trace_obj])
    workers = min(len(cmds), max(1, (os.cpu_count() or 4)))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    os.replace(probe_tmp, PROBE_LIB)
    tmp = LIB + ".tmp"
    _run([cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    trace_objs = [trace_obj if o.endswith("pkv_decode.o") else o for o in objs]
    _run([cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *trace_objs, "-o", TRACE_LIB + ".tmp"],
         verbose)
    os.replace(TRACE_LIB + ".tmp", TRACE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
