"""Compile the gfx950 HIP library (``libfp8qg.so``) in-tree with hipcc.

Every ``csrc/*.hip`` file is compiled to an object (in parallel) and linked into one shared
library next to this file.  No fast-math: the scale is an IEEE-rounded fp32 division.

The device assembly of each file is kept beside its object and checked: no kernel may use a
generic (flat) memory instruction.  A flat access is routed to LDS or to global memory by the
aperture its base address register falls in, so an address the compiler forms as "base below
the LDS aperture + immediate offset" faults with an aperture violation; every access here is
written against LDS or global memory explicitly.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import re
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(os.path.dirname(HERE), "_build")
LIB = os.path.join(HERE, "libfp8qg.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def common_flags() -> list[str]:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-fno-gpu-rdc", "-I", os.path.join(os.path.dirname(HERE), "include")]


def _compile(src: str, obj: str) -> None:
    cmd = [hipcc(), *common_flags(), "-save-temps=obj", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {os.path.basename(src)}:\n{r.stderr[-6000:]}")


FLAT_INSN = re.compile(r"^\s+flat_(load|store|atomic)\w*\s", re.M)


def device_asm(src_name: str) -> str:
    """Path of the gfx950 assembly the build keeps for csrc/<src_name>.hip."""
    return os.path.join(BUILD_DIR, f"{src_name}-hip-amdgcn-amd-amdhsa-{ARCH}.s")


def check_device_asm(srcs: list[str]) -> None:
    for s in srcs:
        name = os.path.basename(s)[:-4]
        text = open(device_asm(name)).read()
        hits = [m.group(0).strip() for m in FLAT_INSN.finditer(text)]
        if hits:
            raise RuntimeError(f"{name}.hip: generic (flat) memory instructions in device code: "
                               f"{hits[:4]} ({len(hits)} in all)")


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(BUILD_DIR, os.path.basename(s)[:-4] + ".o") for s in srcs]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        list(ex.map(lambda so: _compile(*so), zip(srcs, objs)))
    check_device_asm(srcs)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-6000:]}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
