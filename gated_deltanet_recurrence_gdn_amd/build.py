"""Build libgdn.so (the HIP library behind include/gdn.h) for gfx950.

Every source in csrc/ is compiled with hipcc for gfx950 only, in parallel,
into _build/, then linked into libgdn.so inside the package directory, so the
built library travels with the source tree.  Packed-fp32 instruction
selection is turned off for all device code.

build(debug=True) builds the same sources with -DGDN_DEBUG into
libgdn_debug.so: the kernels' indices into the caller's arrays and the
workspace (staging loads, state rows, node states, outputs, commits, the
prefill's raw loads and workspace blocks) are checked, and one past its
array's end is reported as GDN_ERR_INTERNAL through the call's status word and
clamped into the array (the release build compiles the checks away).  Load it
by setting GDN_LIBRARY to its path.
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
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libgdn.so")
DEBUG_LIB = os.path.join(PKG, "libgdn_debug.so")
ARCH = "gfx950"

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core results in ordinary VGPRs (the kernels fit in 256): no
    # accumulator-register copies around the vector ALU work between products
    "-Xarch_device", "-mllvm=-amdgpu-mfma-vgpr-form",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wall", "-Wno-unused-function",
]


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src: str, extra: list[str], build_dir: str = BUILD) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, *extra, "-x", "hip", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, extra: list[str] | None = None, jobs: int = 8, debug: bool = False) -> str:
    extra = list(extra or []) + (["-DGDN_DEBUG"] if debug else [])
    build_dir = BUILD + ("_debug" if debug else "")
    lib = DEBUG_LIB if debug else LIB
    os.makedirs(build_dir, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(jobs, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra, build_dir), srcs))
    tmp = lib + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib} from {len(srcs)} sources", flush=True)
    return lib


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
