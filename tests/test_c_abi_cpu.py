"""The headers compile as plain C11 (-pedantic -Werror) and the built library
can be called from C: tests/c_abi_check.c, linked against librmsnorm.so and
libhbm_copy.so, exercises every entry point's no-GPU behaviour (status
strings, configuration and workspace queries, argument validation)."""
import os
import shutil
import subprocess

import pytest

from memory_bound_rmsnorm_amd import _build

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_c_program_against_the_headers_and_library(tmp_path):
    for lib in (_build.LIB_RMSNORM, _build.LIB_COPY):
        if not os.path.exists(lib):
            pytest.skip("library not built")
    exe = str(tmp_path / "c_abi_check")
    libdir = os.path.dirname(_build.LIB_RMSNORM)
    cmd = ["gcc", "-std=c11", "-Wall", "-Wextra", "-pedantic", "-Werror", os.path.join(HERE, "c_abi_check.c"),
           "-I", os.path.join(ROOT, "include"), "-L", libdir, "-l:" + os.path.basename(_build.LIB_RMSNORM),
           "-l:" + os.path.basename(_build.LIB_COPY), "-Wl,-rpath," + libdir, "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    lines = dict(l.split() for l in run.stdout.splitlines())
    assert lines["fwd_waves_per_row"] == "8" and lines["bwd_workspace_mib"] == "16"
    assert len(lines) > 25
