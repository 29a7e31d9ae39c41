"""Build libqkprep.so (HIP, gfx950 only) in-tree with hipcc.

Every source is compiled for --offload-arch=gfx950 with packed-fp32
instructions disabled (ordinary scalar fp32 code only), then linked into
one shared library next to this file.  Called by ``__graft_entry__.build()``
and ``python -m paged_kv_cache_token_amd.build``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libqkprep.so")
# (source, object name, extra flags): the norm-rope-append kernel is built
# once per head dim so that its instances compile in parallel
SOURCES = [
    ("qkprep_api.hip", "qkprep_api", []),
    ("nra_kernel.hip", "nra_d64", ["-DQKPREP_NRA_HEAD_DIM=64"]),
    ("nra_kernel.hip", "nra_d128", ["-DQKPREP_NRA_HEAD_DIM=128"]),
    ("nra_kernel.hip", "nra_d256", ["-DQKPREP_NRA_HEAD_DIM=256"]),
    ("mla_kernel.hip", "mla_kernel", []),
]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libqkprep")


def compile_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, "-I", CSRC,
    ]


def build(verbose: bool = False) -> str:
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    cc = hipcc()

    def one(item) -> str:
        src, name, extra = item
        obj = os.path.join(objdir, name + ".o")
        cmd = [cc, *compile_flags(), *extra, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
        return obj

    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
