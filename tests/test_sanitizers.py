"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The library's host code (argument checks, the decode and shared-pass
planners, workspace and pool sizing) is compiled host-only with both
sanitizers, the scheduler likewise with g++, and `sanitize_driver.cpp`
exercises them, including seeded random scheduler workloads with pools small
enough to force preemption. No device code is compiled: an empty GPU binary
stands in for the kernels, which are never launched. Any sanitizer report, or
a failed check in the driver, fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_scatter_amd", "csrc")
INC = os.path.join(ROOT, "include")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
ROCM_LIB = "/opt/rocm/lib"

SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined"]
SAN_GXX = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if not os.path.exists(HIPCC) or shutil.which("g++") is None:
        pytest.skip("hipcc or g++ not available")
    d = tmp_path_factory.mktemp("sanitize")
    empty = d / "empty.hip"
    empty.write_text("\n")
    fatbin = d / "empty.hipfb"
    _run([HIPCC, "-x", "hip", "--offload-arch=gfx950", "--cuda-device-only", "-c", str(empty),
          "-o", str(fatbin)])
    objs, procs = [], []
    for name in ("pkv_api", "pkv_write", "pkv_decode", "pkv_prefill"):
        o = d / f"{name}.o"
        objs.append(str(o))
        procs.append(subprocess.Popen(
            [HIPCC, "-std=c++17", "-O1", "-g", "-fPIC", "--offload-arch=gfx950",
             "--cuda-host-only", "-Xclang", "-fcuda-include-gpubinary", "-Xclang", str(fatbin),
             *SAN_HOST, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-c", os.path.join(CSRC, f"{name}.hip"), "-o", str(o)],
            stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
    for name, src in (("pkv_sched", os.path.join(CSRC, "pkv_sched.cpp")),
                      ("driver", os.path.join(ROOT, "tests", "sanitize_driver.cpp"))):
        o = d / f"{name}.o"
        objs.append(str(o))
        procs.append(subprocess.Popen(
            ["g++", "-std=c++17", "-O1", "-g", "-fPIC", *SAN_GXX, "-I" + INC, "-c", src,
             "-o", str(o)], stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
    for p in procs:
        out, err = p.communicate()
        assert p.returncode == 0, f"{' '.join(p.args)}\n{err[-3000:]}"
    exe = d / "driver"
    _run(["g++", *SAN_GXX, *objs, "-L" + ROCM_LIB, "-lamdhip64", "-Wl,-rpath," + ROCM_LIB,
          "-o", str(exe)])
    return str(exe)


def test_driver_links_the_sanitizer_runtimes(driver):
    libs = _run(["ldd", driver]).stdout
    assert "libasan" in libs and "libubsan" in libs


def test_host_code_is_clean_under_asan_and_ubsan(driver):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([driver], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    assert r.stdout.strip() == "ok"
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
