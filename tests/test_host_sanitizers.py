"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

host_abi_driver.c calls every entry point with arguments that its checks
reject (plus empty no-op calls) and sweeps the workspace-size arithmetic
over extreme shapes; no call reaches a HIP launch, so it runs without a GPU.
It is run twice: built with gcc against the shipped library (statuses
only), and against a copy of the library whose host pass is instrumented
(device code is compiled as usual and never runs here).
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from hierarchical_index_sparse_amd import _lib, build_lib

HERE = os.path.dirname(os.path.abspath(__file__))
DRIVER = os.path.join(HERE, "host_abi_driver.c")
CLANG = "/opt/rocm/llvm/bin/clang"
# host pass only: each sanitizer flag goes to the host compiler
HOST_SAN = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined".split()
HOST_SAN += "-Xarch_host -fno-sanitize-recover=undefined -Xarch_host -fno-omit-frame-pointer".split()


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_driver_against_the_library(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    _lib.load()
    lib_dir = os.path.dirname(_lib.LIB_PATH)
    exe = str(tmp_path / "drv")
    _run([gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", build_lib.INCLUDE, DRIVER, "-L", lib_dir,
          "-lhsa_sparse", f"-Wl,-rpath,{lib_dir}", "-Wl,--allow-shlib-undefined", "-o", exe], timeout=120)
    r = _run([exe], timeout=60)
    assert r.stdout.strip().splitlines()[-1].startswith("ok ")


def test_driver_under_host_sanitizers(tmp_path):
    if not (os.path.exists(build_lib.HIPCC) and os.path.exists(CLANG)):
        pytest.skip("no ROCm toolchain")

    def compile_one(src):
        obj = str(tmp_path / (os.path.splitext(src)[0] + ".o"))
        flags = [f for f in build_lib.COMMON_FLAGS if f != "-O3"]
        cmd = [build_lib.HIPCC, *(["-x", "hip"] if src.endswith(".cpp") else []), *flags, "-O1", "-g",
               *HOST_SAN, "-c", os.path.join(build_lib.CSRC, src), "-o", obj]
        _run(cmd, timeout=600)
        return obj

    with ThreadPoolExecutor(min(8, len(build_lib.SOURCES))) as ex:
        objs = list(ex.map(compile_one, build_lib.SOURCES))
    lib = str(tmp_path / "libhsa_sparse_san.so")
    _run([build_lib.HIPCC, f"--offload-arch={build_lib.ARCH}", "-shared", "-fPIC", "-o", lib, *objs], timeout=300)
    exe = str(tmp_path / "drv_san")
    # the executable carries the sanitizer runtimes the library's host code calls into
    _run([CLANG, "-std=c99", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-I",
          build_lib.INCLUDE, DRIVER, "-L", str(tmp_path), "-lhsa_sparse_san", f"-Wl,-rpath,{tmp_path}", "-o", exe],
         timeout=120)
    env = dict(os.environ)
    # the HIP runtime keeps process-lifetime allocations: leak reports off
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1"
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0 and "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr, (
        r.stdout + r.stderr)
    assert r.stdout.strip().splitlines()[-1].startswith("ok ")
