"""The in-launch merge of the decode kernel relies on how gfx950 code
executes its relaxed agent-scope atomics (stated at the merge in
pkv_decode.hip). This compiles the very helpers the kernel uses
(pkv_internal.h) for gfx950 with the library's flags and checks the lowering
the merge depends on, so a toolchain that lowers them otherwise fails here
instead of corrupting results: stores and loads carry sc1 (written through /
not served stale from an XCD's L2), the counter is a returning atomic add, and
no cache-wide write-back or invalidate is emitted. No GPU needed."""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "paged_kv_cache_scatter_amd", "csrc", "pkv_internal.h")
HIPCC = "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else shutil.which("hipcc")

SRC = f"""
#include "{HEADER}"
// results leave through 8-byte stores, so every 4-byte store is the helper's
__global__ void merge_ops(float* p, int* c, double* o) {{
  pkv::dev::st_agent(p + threadIdx.x, (float)threadIdx.x);
  o[threadIdx.x] = pkv::dev::ld_agent(p + 64 + threadIdx.x);
  const float2 v = pkv::dev::ld_agent2(p + 128 + 2 * threadIdx.x);
  o[64 + threadIdx.x] = (double)v.x + v.y;
  if (threadIdx.x == 0) o[200] = (double)pkv::dev::count_agent(c);
}}
"""


@pytest.mark.skipif(HIPCC is None, reason="hipcc not installed")
def test_agent_scope_helpers_lower_as_the_merge_assumes(tmp_path):
    src = tmp_path / "merge_ops.hip"
    src.write_text(SRC)
    asm = tmp_path / "merge_ops.s"
    r = subprocess.run([HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "--cuda-device-only",
                        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-S",
                        str(src), "-o", str(asm)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    text = asm.read_text()
    body = text[text.index("merge_ops"):]
    body = body[:body.index(".Lfunc_end")]
    ops = [ln.strip() for ln in body.splitlines() if ln.strip().startswith(("global_", "buffer_",
                                                                           "flat_"))]
    bits = lambda op: set(re.findall(r"\b(sc0|sc1|nt)\b", op))
    stores = [o for o in ops if o.startswith("global_store_dword ")]
    loads = [o for o in ops if o.startswith(("global_load_dword ", "global_load_dwordx2 "))]
    adds = [o for o in ops if o.startswith("global_atomic_add")]
    assert stores and all("sc1" in bits(o) for o in stores), stores
    assert len(loads) >= 2 and all("sc1" in bits(o) for o in loads), loads
    assert len(adds) == 1 and "sc0" in bits(adds[0]), adds     # returns the old count
    assert not any(o.startswith(("buffer_wbl2", "buffer_inv")) for o in ops), ops
