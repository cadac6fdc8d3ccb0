"""Build libmla.so (HIP kernels + C ABI) in-tree for gfx950 with hipcc.

    python -m mla_latent_kv_23_amd.build

Every call recompiles; objects go to mla_latent_kv_23_amd/_build/, the shared
library to mla_latent_kv_23_amd/libmla.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmla.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmla)")


COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


# AddressSanitizer on the host code only (argument checks, planning, the ABI
# layer); the device code is compiled as usual.  Load the result with the
# clang ASan runtime preloaded (see asan_runtime()).
ASAN_FLAGS = ["-O1", "-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
ASAN_BUILD = os.path.join(BUILD, "asan")
ASAN_LIB = os.path.join(ASAN_BUILD, "libmla_asan.so")


def asan_runtime() -> str:
    """The clang AddressSanitizer runtime that matches hipcc's compiler."""
    found = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not found:
        raise RuntimeError("clang AddressSanitizer runtime not found under /opt/rocm/lib/llvm")
    return found[-1]


def _compile(src: str, out_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMMON, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


def build_asan(verbose: bool = False) -> str:
    """libmla_asan.so: the library with its host code under AddressSanitizer
    (a checker of the host layer; the product library is build())."""
    os.makedirs(ASAN_BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda f: _compile(f, ASAN_BUILD, ASAN_FLAGS), srcs))
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address", "-o",
           ASAN_LIB, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(f"built {ASAN_LIB} from {len(srcs)} sources")
    return ASAN_LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
