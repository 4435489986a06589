"""Build libpgqa.so (gfx950) in-tree with hipcc.

    python -m paged_gqa_decode_head_amd.build [-v]

Each translation unit is compiled to an object in ``_build/`` (in parallel) and
linked into ``paged_gqa_decode_head_amd/libpgqa.so``.  Every call rebuilds.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpgqa.so")

SOURCES = ["errors.cpp", "api.cpp", "sched.cpp", "cache_write.hip", "decode.hip", "chunk.hip", "mixed.hip",
           "stream_read.hip"]

ARCH = "gfx950"
COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    f"-I{os.path.join(ROOT, 'include')}",
]
# Packed fp32 VALU forms are kept out of the device code.
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# Per-file device options.  chunk.hip, mixed.hip: MFMA accumulators in VGPRs
# rather than AGPRs (the narrow kernel otherwise copies them between the
# register files around every softmax rescale).
EXTRA = {"chunk.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"], "mixed.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libpgqa")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    path = os.path.join(CSRC, src)
    cmd = [hipcc(), *COMMON, *DEVICE, *EXTRA.get(src, []), "-c", path, "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = ["-x", "hip"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking libpgqa.so failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    build_c_consumer(verbose)
    return LIB


def build_c_consumer(verbose: bool = False) -> str:
    """tests/c_decode_step.c (the C-ABI decode step driven from C with the HIP
    runtime) -> tests/bin/c_decode_step, linked to the in-tree libpgqa.so."""
    src = os.path.join(ROOT, "tests", "c_decode_step.c")
    out = os.path.join(ROOT, "tests", "bin", "c_decode_step")
    if not os.path.exists(src):
        return ""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no C compiler found for tests/c_decode_step.c")
    cmd = [cc, "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           f"-I{os.path.join(rocm, 'include')}", f"-I{os.path.join(ROOT, 'include')}", src,
           f"-L{PKG}", "-lpgqa", f"-L{os.path.join(rocm, 'lib')}", "-lamdhip64",
           f"-Wl,-rpath,{os.path.join(rocm, 'lib')}", "-Wl,-rpath,$ORIGIN/../../paged_gqa_decode_head_amd", "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"building {src} failed:\n{r.stdout}\n{r.stderr}")
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
