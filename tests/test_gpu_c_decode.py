"""The C ABI from plain C on the GPU: tests/c_decode.c (C11, HIP runtime C
API for device memory, no C++ and no PyTorch) is built with gcc against
include/pkv.h and libpkv.so and runs decode steps whose result has a closed
form (a zero query: every output channel is the mean of the row's value
codes times v_scale, lse = log(len)), with the automatic geometry (one
split, direct output) and with three splits (the combine), and checks that a
too-small workspace is refused."""
import os
import shutil
import subprocess

import pytest

from tests.gpu_util import announce

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def test_plain_c_program_decodes_on_the_gpu(tmp_path):
    import quantized_paged_kv_amd as pkv

    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    libdir = os.path.dirname(pkv.LIB_PATH)
    exe = str(tmp_path / "c_decode")
    subprocess.run([gcc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c_decode.c"), "-L", libdir, "-lpkv",
                    "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
                    f"-Wl,-rpath,{libdir}", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", exe],
                   check=True)
    announce("plain C decode program")
    res = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, (res.returncode, res.stdout, res.stderr)
    assert res.stdout.strip().endswith("ok"), res.stdout
