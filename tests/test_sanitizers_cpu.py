"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

- The oracle: tests/c_oracle_sanitize.c drives every oracle function on
  exactly sized buffers (gcc, -fsanitize=address,undefined,float-cast-overflow).
- The C-ABI library's host code (argument validation, launch-shape choice,
  workspace sizing): every source is compiled host-only with the sanitizers
  (device code is not built, so nothing can be launched), linked into a
  library that tests/c_abi_sweep.c and tests/c_abi_check.c call with fake
  device addresses.  Sanitizer reports end the programs with an error
  (-fno-sanitize-recover=all).
"""
import concurrent.futures
import os
import shutil
import subprocess

import pytest

from memory_bound_rmsnorm_amd import _build

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CLANG = os.path.join(_build.ROCM, "llvm", "bin", "clang")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
# each sanitizer flag follows -Xarch_host, so that it applies to host code only
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    p = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert p.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), p.stdout[-3000:], p.stderr[-3000:])
    return p


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    _run(["gcc", "-std=c99", "-O1", "-g", "-fsanitize=address,undefined,float-cast-overflow",
          "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-ffp-contract=off", "-Wall", "-Wextra",
          "-Werror", os.path.join(HERE, "c_oracle_sanitize.c"), os.path.join(ROOT, "oracle", "rmsnorm_oracle.c"),
          "-lm", "-o", exe])
    p = _run([exe], env=ENV, timeout=300)
    assert "0 failures" in p.stdout


@pytest.mark.skipif(not (os.path.exists(_build.HIPCC) and os.path.exists(CLANG)), reason="no ROCm toolchain")
def test_library_host_code_under_sanitizers(tmp_path):
    def compile_one(src):
        obj = str(tmp_path / (os.path.splitext(src)[0] + ".o"))
        _run([_build.HIPCC, "--offload-arch=" + _build.ARCH, "-fgpu-rdc", "--cuda-host-only", "-O1", "-g",
              "-std=c++17", "-fPIC", "-fvisibility=hidden"] + HOST_SANITIZE +
             ["-c", os.path.join(_build.CSRC, src), "-o", obj])
        return obj

    sources = _build.RMSNORM_SOURCES + _build.COPY_SOURCES
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 4)) as ex:
        objs = list(ex.map(compile_one, sources))
    lib = str(tmp_path / "libabi_sanitized.so")
    _run([_build.HIPCC, "--offload-arch=" + _build.ARCH, "-fgpu-rdc", "-shared", "-fPIC"] + HOST_SANITIZE[:4] +
         ["-o", lib] + objs)
    for driver, want in (("c_abi_sweep.c", "0 failures"), ("c_abi_check.c", "copy_null")):
        exe = str(tmp_path / os.path.splitext(driver)[0])
        _run([CLANG, "-std=c11", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
              "-fno-omit-frame-pointer", "-Wall", "-Wextra", "-I", os.path.join(ROOT, "include"),
              os.path.join(HERE, driver), "-L", str(tmp_path), "-l:libabi_sanitized.so",
              "-Wl,-rpath," + str(tmp_path), "-Wl,-rpath," + os.path.join(_build.ROCM, "lib"), "-o", exe])
        p = _run([exe], env=ENV, timeout=300)
        assert want in p.stdout, p.stdout[-2000:]
