"""The teacher-cache host code under AddressSanitizer and UndefinedBehaviorSanitizer.

kdcache.cpp (shard files, the loader and the writer) is host code: it is built
here with g++ and both sanitizers (the sanitizers apply to host code only; no
device code is involved) and driven by tests/c_abi/kdcache_check.c, a C program
that runs round trips over both index widths and value types, partial reads,
every argument error, corrupted and truncated files (each header field and the
file size) and the open/close paths of the loader and the writer.  Any invalid
memory access, leak or undefined operation makes the program fail.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g", "-O1"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)} -> {r.returncode}\n{r.stdout[-4000:]}"
    return r.stdout


@pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None
                    or not os.path.exists(os.path.join(ROCM, "lib", "libamdhip64.so")),
                    reason="needs gcc, g++ and the HIP runtime library")
def test_cache_host_code_under_sanitizers(tmp_path):
    inc = ["-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include")]
    lib = os.path.join(tmp_path, "kdcache.o")
    drv = os.path.join(tmp_path, "check.o")
    exe = os.path.join(tmp_path, "kdcache_check")
    _run(["g++", "-std=c++17", "-Wall", "-Wextra", "-Werror", *SAN, *inc, "-c",
          os.path.join(ROOT, "lm_head_kl_amd", "csrc", "kdcache.cpp"), "-o", lib])
    _run(["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", *SAN, *inc, "-c",
          os.path.join(ROOT, "tests", "c_abi", "kdcache_check.c"), "-o", drv])
    _run(["g++", *SAN, drv, lib, "-L", os.path.join(ROCM, "lib"), f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}",
          "-lamdhip64", "-lpthread", "-o", exe])
    scratch = tmp_path / "scratch"
    scratch.mkdir()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    out = _run([exe, str(scratch)], env=env, timeout=300)
    assert out.strip().startswith("ok "), out
    assert int(out.split()[1]) > 1000
