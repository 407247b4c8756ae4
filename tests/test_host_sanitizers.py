"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Every library source is compiled with the sanitizers on its host side only
(`-Xarch_host`; device code is built as in the product), a host-only driver
(tests/sanitize/abi_host_driver.cpp) is compiled with them too, and the two
are linked with clang++. The driver runs every entry-point path that returns
before a HIP call (argument checks, the workspace plan over the size
envelope, status strings, the workspace check), so no GPU is needed. A
sanitizer report aborts the driver (no recovery) and fails the test.
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from aware_expert_routing_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang++"
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


@pytest.mark.skipif(not (os.path.exists("/opt/rocm/bin/hipcc") and os.path.exists(CLANG)),
                    reason="ROCm compilers not installed")
def test_abi_host_paths_under_asan_and_ubsan(tmp_path):
    host_san = [f for flag in SAN for f in ("-Xarch_host", flag)]

    def compile_src(src):
        obj = str(tmp_path / (os.path.splitext(src)[0] + ".o"))
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [B._hipcc(), "-O1", "-g", "-std=c++17", "-fPIC", f"--offload-arch={B.ARCH}", *B.DEVICE_FLAGS,
               *host_san, *lang, "-c", os.path.join(B.CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return obj

    with ThreadPoolExecutor(max_workers=min(8, len(B.SOURCES))) as ex:
        objs = list(ex.map(compile_src, B.SOURCES))
    drv = str(tmp_path / "driver.o")
    r = subprocess.run([CLANG, "-O1", "-g", "-std=c++17", *SAN, "-I", os.path.join(ROOT, "include"), "-c",
                        os.path.join(ROOT, "tests", "sanitize", "abi_host_driver.cpp"), "-o", drv],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    exe = str(tmp_path / "driver")
    r = subprocess.run([CLANG, "-fsanitize=address,undefined", *objs, drv, "-L/opt/rocm/lib", "-lamdhip64",
                        "-Wl,-rpath,/opt/rocm/lib", "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "0 failures" in r.stdout
