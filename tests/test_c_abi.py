"""The C ABI from plain C: tests/c/abi_demo.c is compiled with gcc against
include/tsp_mlp.h and the built library (CPU: compile and link only; GPU: run
it and check its outputs)."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c", "abi_demo.c")
LIBDIR = os.path.join(ROOT, "sharded_transformer_mlp_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(tmp_path):
    exe = str(tmp_path / "abi_demo")
    cmd = ["gcc", "-std=c11", "-O1", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), SRC, "-o", exe,
           "-L", LIBDIR, "-ltsp_mlp", "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
           f"-Wl,-rpath,{LIBDIR}", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return exe


def test_c_program_compiles_and_links(tmp_path):
    if not os.path.exists(os.path.join(LIBDIR, "libtsp_mlp.so")):
        pytest.skip("library not built")
    assert os.path.exists(build(tmp_path))


@pytest.mark.gpu
def test_c_program_runs(tmp_path):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    exe = build(tmp_path)
    for T in (1, 40, 300):
        r = subprocess.run([exe, str(T)], capture_output=True, text=True, timeout=120)
        print(r.stdout.strip(), r.stderr.strip(), flush=True)
        assert r.returncode == 0, r.stdout + r.stderr

