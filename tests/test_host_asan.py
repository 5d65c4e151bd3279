"""Host AddressSanitizer build of the C ABI's planning code, CPU only: capi.cpp
(tree validation, the metadata plan, capacity checks) is recompiled with the
host pass instrumented (hipcc -Xarch_host -fsanitize=address; device code is
built as usual) and linked with the other objects of the library into a
separate copy of it; tests/asan_plan_driver.py then runs every planning entry
point in a child process with the sanitizer runtime preloaded (exact-size
staging buffers, exact capacities, rejection paths). Any out-of-bounds access
or use after free in the host code aborts the child."""
import glob
import os
import subprocess
import sys

import pytest

from tree_structured_decision_amd import build as hb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def asan_runtime():
    c = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return c[-1] if c else None


@pytest.mark.timeout(600)
def test_plan_code_under_address_sanitizer():
    rt = asan_runtime()
    if rt is None:
        pytest.skip("clang AddressSanitizer runtime not found")
    out = os.path.join(hb.BUILD_DIR, "asan")
    os.makedirs(out, exist_ok=True)
    objs = []
    for src in hb.SOURCES:
        if src == "capi.cpp":
            continue
        o = os.path.join(hb.BUILD_DIR, os.path.splitext(src)[0] + ".o")
        objs.append(o if os.path.exists(o) else hb._compile(src))
    capi = os.path.join(out, "capi_asan.o")
    cmd = [hb.hipcc()] + hb.common_flags() + ["-Xarch_host", "-fsanitize=address",
                                               "-Xarch_host", "-fno-omit-frame-pointer", "-x", "hip", "-c",
                                               os.path.join(hb.CSRC, "capi.cpp"), "-o", capi]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    lib = os.path.join(out, "libforkattn_asan.so")
    cmd = [hb.hipcc(), f"--offload-arch={hb.ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
           "-shared-libasan", "-o", lib, capi] + objs + ["-lhipblaslt"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    # the plan code calls into the sanitizer (its accesses are checked)
    r = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True)
    assert "__asan_report_load4" in r.stdout and "__asan_report_store4" in r.stdout
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               PYTHONPATH=ROOT + os.pathsep + os.environ.get("PYTHONPATH", ""))
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "asan_plan_driver.py"), lib],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=500)
    assert "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "asan driver:" in r.stdout
    print(r.stdout.strip())
