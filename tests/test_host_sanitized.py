"""The libraries' host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The sanitizers apply to host code only; no device code is built or run here.

* kdcache.cpp (shard files, the loader and the writer) is built with g++ and
  driven by tests/c_abi/kdcache_check.c: round trips over both index widths and
  value types, partial reads, every argument error, corrupted and truncated files
  (each header field and the file size) and the open/close paths of the loader
  and the writer.
* kdkl.hip is built with the library's flags plus the host-side sanitizers and driven by
  tests/c_abi/kdkl_check.c: the workspace size over a product of shapes at and
  past every domain limit, checked against the header's domain, and the argument
  errors of every entry point, none of which reaches the device.

* kdcache.cpp again, with tests/c_abi/hip_host_stub.cpp in place of the HIP
  runtime (host memory for pinned and device buffers, copies at once), so that
  the writer's and loader's background threads run here: under ThreadSanitizer,
  then AddressSanitizer, driven by tests/c_abi/kdcache_threads.c (uneven batches
  into shards, loading across shard boundaries, the writer's failure path, a
  loader closed mid-stream, four writer/loader pairs at once).

Any invalid memory access, leak, data race or undefined operation (signed
overflow in the size arithmetic included) makes a program fail.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g", "-O1"]
# the same for hipcc, each sanitizer flag for the host side only
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)} -> {r.returncode}\n{r.stdout[-4000:]}"
    return r.stdout


needs_tools = pytest.mark.skipif(
    shutil.which("g++") is None or shutil.which("gcc") is None
    or not os.path.exists(os.path.join(ROCM, "lib", "libamdhip64.so")),
    reason="needs gcc, g++ and the HIP runtime library")


def _link_and_run(tmp_path, objs, args):
    exe = os.path.join(tmp_path, "check")
    _run(["g++", *SAN, *objs, "-L", os.path.join(ROCM, "lib"), f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}",
          "-lamdhip64", "-lpthread", "-lm", "-o", exe])
    out = _run([exe, *args], env=ENV, timeout=300)
    assert out.strip().startswith("ok "), out
    return int(out.split()[1])


@needs_tools
def test_cache_host_code_under_sanitizers(tmp_path):
    inc = ["-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include")]
    lib = os.path.join(tmp_path, "kdcache.o")
    drv = os.path.join(tmp_path, "check.o")
    _run(["g++", "-std=c++17", "-Wall", "-Wextra", "-Werror", *SAN, *inc, "-c",
          os.path.join(ROOT, "lm_head_kl_amd", "csrc", "kdcache.cpp"), "-o", lib])
    _run(["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", *SAN, *inc, "-c",
          os.path.join(ROOT, "tests", "c_abi", "kdcache_check.c"), "-o", drv])
    scratch = tmp_path / "scratch"
    scratch.mkdir()
    assert _link_and_run(tmp_path, [drv, lib], [str(scratch)]) > 1000


@needs_tools
def test_loss_library_host_code_under_sanitizers(tmp_path):
    from lm_head_kl_amd import build
    inc = ["-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include")]
    lib = os.path.join(tmp_path, "kdkl.o")
    drv = os.path.join(tmp_path, "check.o")
    # the library's own flags (device code included, as it links only with its code
    # object), with the sanitizers added for the host side
    # (the loaders' inline asm names the reserved M0 register as clobbered, on purpose)
    flags = [f for f in build.HIPCC_FLAGS if f != "-shared"]
    _run([build.hipcc(), "-x", "hip", *flags, "-Wall", "-Werror", "-Wno-inline-asm", *HOST_SAN,
          "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "lm_head_kl_amd", "csrc"), "-c",
          os.path.join(ROOT, "lm_head_kl_amd", "csrc", "kdkl.hip"), "-o", lib])
    _run(["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", *SAN, *inc, "-c",
          os.path.join(ROOT, "tests", "c_abi", "kdkl_check.c"), "-o", drv])
    assert _link_and_run(tmp_path, [drv, lib], []) > 1_000_000


@pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None, reason="needs gcc and g++")
@pytest.mark.parametrize("san", ["thread", "address,undefined"])
def test_cache_threads_under_sanitizers(tmp_path, san):
    inc = ["-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include")]
    flags = [f"-fsanitize={san}", "-fno-omit-frame-pointer", "-g", "-O1", "-Wall", "-Wextra", "-Werror"]
    objs = []
    for src, cc, std in ((os.path.join("lm_head_kl_amd", "csrc", "kdcache.cpp"), "g++", "c++17"),
                         (os.path.join("tests", "c_abi", "hip_host_stub.cpp"), "g++", "c++17"),
                         (os.path.join("tests", "c_abi", "kdcache_threads.c"), "gcc", "c11")):
        obj = os.path.join(tmp_path, os.path.basename(src) + ".o")
        _run([cc, f"-std={std}", *flags, *inc, "-c", os.path.join(ROOT, src), "-o", obj])
        objs.append(obj)
    exe = os.path.join(tmp_path, "threads")
    _run(["g++", f"-fsanitize={san}", *objs, "-lpthread", "-o", exe])
    scratch = tmp_path / "scratch"
    scratch.mkdir()
    env = dict(ENV, TSAN_OPTIONS="halt_on_error=1:second_deadlock_stack=1")
    out = _run([exe, str(scratch)], env=env, timeout=300)
    assert out.strip().startswith("ok "), out
