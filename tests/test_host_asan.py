"""Host code under AddressSanitizer (CPU only): tests/c/abi_validate.c walks
every host-side error path of the C ABI against a copy of the library whose
host code is built with ASan (the device passes are built as usual; the
sanitizer flag is given to the host pass only), with leak detection on."""
import glob
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

ASAN_SRC = os.path.join(ROOT, "tests", "c", "abi_validate.c")
CSRC = os.path.join(ROOT, "sharded_transformer_mlp_amd", "csrc")


def test_host_error_paths_under_address_sanitizer(tmp_path):
    clang = os.path.join(ROCM, "llvm", "bin", "clang")
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    if not (os.path.exists(clang) and os.path.exists(hipcc)):
        pytest.skip("ROCm compilers not found")
    # the library's host code with ASan: api.hip holds all of it (the other
    # sources only add kernels and their launchers)
    objs = []
    for src in sorted(f for f in os.listdir(CSRC) if f.endswith(".hip")):
        obj = str(tmp_path / (src + ".o"))
        flags = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"] \
            if src == "api.hip" else []
        subprocess.run([hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", *flags,
                        "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj],
                       check=True, capture_output=True, text=True)
        objs.append(obj)
    lib = str(tmp_path / "libtsp_mlp_asan.so")
    subprocess.run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
                    "-shared-libsan", *objs, "-o", lib], check=True, capture_output=True, text=True)
    rt = glob.glob(os.path.join(ROCM, "llvm", "lib", "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so"))
    if not rt:
        pytest.skip("clang ASan runtime not found")
    rtdir = os.path.dirname(rt[0])
    exe = str(tmp_path / "abi_validate")
    subprocess.run([clang, "-std=c11", "-O1", "-g", "-Wall", "-Werror", "-fsanitize=address", "-shared-libsan",
                    "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
                    ASAN_SRC, "-o", exe, lib, f"-Wl,-rpath,{tmp_path}", f"-Wl,-rpath,{rtdir}", "-L", os.path.join(ROCM, "lib"),
                    "-lamdhip64", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"],
                   check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout + r.stderr[-4000:]
    assert "0 failure(s)" in r.stdout
    assert "ERROR: AddressSanitizer" not in r.stderr
