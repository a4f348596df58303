"""Builds libtsp_mlp.so (the C-ABI library) from csrc/*.hip for gfx950.

Usage: ``python -m sharded_transformer_mlp_amd.build``. Objects go to
``_build/`` at the repository root; the shared library lands next to this
file, where the binding loads it.
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libtsp_mlp.so")
# Same sources with TSP_LDS_POISON: every kernel fills its LDS with NaN
# before first use (tests run parity cases on it to catch missing waits).
DEBUG_LIB = os.path.join(PKG, "libtsp_mlp_lds_poison.so")
ARCH = "gfx950"

# Packed-fp32 VALU ops are disabled for every device pass.
HIPFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


# Per-source codegen options: the attention kernel keeps its MFMA results in
# vector registers (its softmax reads every score; results in accumulation
# registers were copied out one by one). Other scheduling strategies than the
# default measured no gain or spilled registers, for the attention kernel at
# two waves per SIMD and for the fenced 256 x 256 kernels.
EXTRA_FLAGS = {"attn_core.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


# Every kernel's register use is reported by the compiler; a kernel that
# needs scratch memory (registers spilled to memory) fails the build: such a
# spill once came with wrong accumulator values, and it always costs memory
# traffic in the hot loops. Spills into free accumulation registers use no
# memory and are allowed.
RESOURCE_REMARKS = ["-Rpass-analysis=kernel-resource-usage", "-fno-caret-diagnostics"]


def _check_spills(src: str, remarks) -> None:
    fn, bad = None, []
    for line in remarks:
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            fn = m.group(1)
            continue
        m = re.search(r"(ScratchSize \[bytes/lane\]): (\d+)", line)
        if m and int(m.group(2)) > 0:
            bad.append(f"{fn}: {m.group(1)} {m.group(2)}")
    if bad:
        raise RuntimeError(f"{src}: kernels use scratch memory:\n  " + "\n  ".join(bad))


def _compile(src: str, tag: str = "", defs=()) -> str:
    obj = os.path.join(OBJ, os.path.basename(src) + tag + ".o")
    cmd = [hipcc(), *HIPFLAGS, *RESOURCE_REMARKS, *EXTRA_FLAGS.get(os.path.basename(src), []), *defs, "-c", src,
           "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    lines = [l for l in r.stderr.splitlines() if noise not in l]
    remarks = [l for l in lines if "kernel-resource-usage" in l]
    err = "\n".join(l for l in lines if "kernel-resource-usage" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    _check_spills(src, remarks)
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def _link(objs, out: str) -> None:
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = True) -> str:
    """Compile every source and link the shared library (and its LDS-poison
    debug twin); returns the library's path."""
    os.makedirs(OBJ, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max_workers=min(8, 2 * len(srcs))) as ex:
        objs = ex.map(_compile, srcs)
        dbg = ex.map(lambda s: _compile(s, ".poison", ("-DTSP_LDS_POISON=1",)), srcs)
        objs, dbg = list(objs), list(dbg)
    _link(objs, LIB)
    _link(dbg, DEBUG_LIB)
    if verbose:
        print(f"built {LIB} and {os.path.basename(DEBUG_LIB)} from {len(srcs)} sources")
    return LIB


if __name__ == "__main__":
    build()
