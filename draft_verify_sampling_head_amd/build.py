"""Build libdspark.so (HIP, gfx950) in-tree with hipcc.

Every .hip source under csrc/ is compiled to an object in parallel, then the
objects are linked into draft_verify_sampling_head_amd/libdspark.so.  Packed
fp32 instructions are disabled for all device code.
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
OBJDIR = os.path.join(ROOT, "_build", "obj")
LIB = os.path.join(PKG, "libdspark.so")
ARCH = os.environ.get("DSPARK_ARCH", "gfx950")

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-ffp-contract=fast", "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def rocm_lib() -> str:
    """The ROCm library folder next to the hipcc in use."""
    return os.path.join(os.path.dirname(os.path.dirname(hipcc())), "lib")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libdspark.so")


# roctx (marker ranges around each C-ABI call)
def _link_flags() -> list:
    lib = rocm_lib()
    return [f"-L{lib}", "-lrocprofiler-sdk-roctx", f"-Wl,-rpath,{lib}"]


def _compile(src: str, objdir: str = OBJDIR, extra: tuple = ()) -> str:
    obj = os.path.join(objdir, os.path.basename(src).replace(".hip", ".o"))
    cmd = [hipcc()] + FLAGS + list(extra) + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, lib_path: str = LIB, objdir: str = OBJDIR,
          extra_flags: tuple = ()) -> str:
    """Compile every source and link lib_path.  extra_flags go to every
    compile line (another build of the same sources, e.g. with host-only
    instrumentation, into its own objdir and lib_path)."""
    os.makedirs(objdir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    workers = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(lambda s: _compile(s, objdir, tuple(extra_flags)), srcs))
    tmp = lib_path + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs + _link_flags()
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib_path)
    if verbose:
        print(f"built {lib_path}")
    return lib_path


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
