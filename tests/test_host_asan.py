"""Host-side argument checks of the C ABI under AddressSanitizer.

The library's host code (every entry point's rejections, the workspace size
computations, the host validators) is rebuilt with AddressSanitizer on the
host side only (device code is compiled as usual and never run here), linked
with tests/asan_host_checks.cpp, and run on the CPU: no call in the driver
reaches a launch. Arrays are sized exactly, so a read past an argument
fails the run.
"""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "tree_verification_verify_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
SOURCES = ["tree_attn.hip", "tree_sample.hip", "tree_sample_noalloc.hip", "tree_path.hip",
           "tree_commit.hip", "tree_siblings.hip", "tree_construct.hip", "tree_spark.hip", "api.cpp"]


def _hipcc():
    for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc") or ""):
        if c and os.path.exists(c):
            return c
    return None


@pytest.mark.timeout(600)
def test_host_checks_under_address_sanitizer():
    cc = _hipcc()
    if cc is None:
        pytest.skip("hipcc not available")
    # the sanitizer applies to host code only: each -fsanitize flag follows -Xarch_host
    host_asan = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
    base = ["-O1", "-g", "-std=c++17", "-I", INCLUDE, "-I", CSRC]
    with tempfile.TemporaryDirectory() as d:
        procs, objs = [], []
        for src in SOURCES:
            obj = os.path.join(d, os.path.splitext(src)[0] + ".o")
            cmd = [cc, "--offload-arch=gfx950"] + base + host_asan
            if src.endswith(".cpp"):
                cmd += ["-x", "hip"]
            cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
            objs.append(obj)
        for src, pr in procs:
            out = pr.communicate()[0]
            assert pr.returncode == 0, (src, out.decode()[-2000:])
        drv = os.path.join(d, "drv.o")
        r = subprocess.run([cc] + base + ["-Xarch_host", "-fsanitize=address", "-c",
                            os.path.join(ROOT, "tests", "asan_host_checks.cpp"), "-o", drv],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        exe = os.path.join(d, "asan_host_checks")
        r = subprocess.run([cc, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address"] + objs +
                           [drv, "-o", exe], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        nm = subprocess.run(["nm", exe], capture_output=True, text=True).stdout
        assert "__asan_init" in nm or "__asan_report" in nm  # the host code is instrumented
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0")
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
        assert "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
        assert r.returncode == 0 and "ok (0 failures)" in r.stdout, (r.stdout[-2000:], r.stderr[-2000:])
