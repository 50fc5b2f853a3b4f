"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).

Every library source is compiled with the sanitizers applied to host code only
(``-Xarch_host``; device code is built as usual and never runs here), linked
with ``abi_asan_driver.c``, and run.  The driver calls every entry point through
its validation paths with fake pointers and checks the documented status
codes, enumerates the W4A16 selector and checks the per-thread error message.
A sanitizer report or a failed check makes the driver exit non-zero."""

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from block_scaled_precision_bsgemm_amd import build as B

HERE = os.path.dirname(os.path.abspath(__file__))
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]


def _hipcc():
    path = "/opt/rocm/bin/hipcc"
    return path if os.path.exists(path) else shutil.which("hipcc")


@pytest.mark.skipif(_hipcc() is None, reason="hipcc is not installed")
def test_host_code_under_sanitizers(tmp_path):
    import torch
    if torch.cuda.is_available():
        pytest.skip("host-side sanitizer run: meant for machines without a GPU")
    hipcc = _hipcc()
    flags = ["-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
             "-I" + B.INCLUDE, "-I" + B.CSRC, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"] + SAN

    def compile_one(src):
        out = str(tmp_path / (src + ".o"))
        r = subprocess.run([hipcc] + flags + ["-c", os.path.join(B.CSRC, src), "-o", out],
                           capture_output=True, text=True)
        assert r.returncode == 0, f"{src}:\n{r.stderr[-3000:]}"
        return out

    with ThreadPoolExecutor(max_workers=min(len(B.SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, B.SOURCES))
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc)), "..", "lib", "llvm", "bin", "clang")
    clang = clang if os.path.exists(clang) else "clang"
    drv = str(tmp_path / "driver.o")
    r = subprocess.run([clang, "-O1", "-g", "-fsanitize=address,undefined", "-I" + B.INCLUDE, "-c",
                        os.path.join(HERE, "abi_asan_driver.c"), "-o", drv], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    exe = str(tmp_path / "driver")
    r = subprocess.run([hipcc, "--offload-arch=gfx950"] + SAN + objs + [drv, "-o", exe, "-lpthread"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="halt_on_error=1:detect_leaks=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe, "--no-gpu"], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, f"driver failed ({r.returncode}):\n{r.stdout[-2000:]}\n{r.stderr[-4000:]}"
    assert "all checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
