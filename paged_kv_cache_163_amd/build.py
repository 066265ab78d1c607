"""Build libpa.so (the C-ABI library of HIP kernels) for gfx950, in-tree.

    python -m paged_kv_cache_163_amd.build

Each ``csrc/*.hip`` is compiled with hipcc and each host-only ``csrc/*.cpp``
with the host C++ compiler, in parallel, then linked into
``paged_kv_cache_163_amd/libpa.so`` (written atomically).  hipcc
cross-compiles for gfx950 without a GPU present.
"""

from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpa.so")
ARCH = "gfx950"

# Packed fp32 VALU ops are disabled: the kernels never rely on them.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra"]


def cxx() -> str:
    for cand in (os.environ.get("CXX"), shutil.which("g++"), shutil.which("c++")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("no host C++ compiler (set CXX)")


# The compiler's per-kernel resource report (registers, scratch, occupancy).
RESOURCE_REMARKS = "-Rpass-analysis=kernel-resource-usage"


def kernel_resources(remarks: str) -> dict:
    """Per-kernel fields of the resource report in a compiler's stderr:
    {kernel symbol: {"VGPRs": int, "ScratchSize [bytes/lane]": int, ...}}."""
    out: dict = {}
    cur = None
    for line in remarks.splitlines():
        if "remark:" not in line or "kernel-resource-usage" not in line:
            continue
        body = line.split("remark:", 1)[1].rsplit("[-Rpass-analysis", 1)[0].strip()
        key, _, val = body.partition(":")
        key, val = key.strip(), val.strip()
        if key == "Function Name":
            cur = out.setdefault(val, {})
        elif cur is not None:
            try:
                cur[key] = int(val)
            except ValueError:
                cur[key] = val
    return out


def _compile(src: str, obj: str) -> None:
    if src.endswith(".cpp"):
        cmd = [cxx(), *HOST_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]
    else:
        cmd = [hipcc(), *HIP_FLAGS, RESOURCE_REMARKS, "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    if src.endswith(".hip"):
        # Every kernel is register-budgeted: a spill to scratch is a build
        # error.  Besides its cost, it would put vector memory operations in
        # the prefill key loop, whose direct LDS staging counts them.
        spilled = {k: v for k, v in kernel_resources(res.stderr).items()
                   if v.get("ScratchSize [bytes/lane]", 0) != 0}
        if spilled:
            raise RuntimeError(f"{os.path.basename(src)}: kernels spill to scratch: {spilled}")


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    objs = [os.path.join(BUILD_DIR, os.path.splitext(os.path.basename(s))[0] + ".o") for s in srcs]
    workers = max(1, min(len(srcs), os.cpu_count() or 1, 8))
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        list(ex.map(_compile, srcs, objs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
