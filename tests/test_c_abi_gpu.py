"""The C-ABI boundary from a plain C11 program on the GPU: tests/c_abi_gpu.c
allocates with the HIP runtime's C API, calls rmsnorm_fwd,
rmsnorm_residual_fwd, rmsnorm_bwd and layernorm_fwd on its own stream, and
checks properties of the results (see the program's header)."""
import os
import shutil
import subprocess

import pytest

from memory_bound_rmsnorm_amd import _build

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.gpu
@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_c_program_on_the_gpu(tmp_path):
    exe = str(tmp_path / "c_abi_gpu")
    libdir = os.path.dirname(_build.LIB_RMSNORM)
    rocm_lib = os.path.join(_build.ROCM, "lib")
    subprocess.run(["gcc", "-std=c11", "-O1", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROOT, "include"), "-I", os.path.join(_build.ROCM, "include"),
                    os.path.join(HERE, "c_abi_gpu.c"), "-L", libdir, "-l:" + os.path.basename(_build.LIB_RMSNORM),
                    "-L", rocm_lib, "-lamdhip64", "-lm", "-Wl,-rpath," + libdir, "-Wl,-rpath," + rocm_lib, "-o", exe],
                   check=True, capture_output=True, text=True)
    print("running", exe, flush=True)
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(run.stdout)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "0 failures" in run.stdout
