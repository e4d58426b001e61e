"""Build libattn.so (the C-ABI attention library) for gfx950 with hipcc.

Usage: python -m tiled_attention_attn_amd.build [--resource-usage]
The library is written next to this file so it travels with the source tree.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJDIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libattn.so")
SOURCES = ["attn_api.hip", "attn_bf16.hip", "attn_f32.hip", "bcast_group.hip", "ikbo_gemm.hip",
           "rmsnorm.hip", "ceiling.hip"]
ARCH = "gfx950"

# Packed fp32 VALU ops are turned off for every HIP translation unit.
HIPFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-result"]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the attention library needs ROCm's hipcc")


def _compile(src: str, extra) -> tuple[str, str]:
    obj = os.path.join(OBJDIR, src.replace(".hip", ".o"))
    cmd = [_hipcc(), *HIPFLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj, r.stderr


def build(resource_usage: bool = False, verbose: bool = False) -> str:
    """Compile every source for gfx950 and link libattn.so; returns its path."""
    os.makedirs(OBJDIR, exist_ok=True)
    extra = ["-Rpass-analysis=kernel-resource-usage"] if resource_usage else []
    with cf.ThreadPoolExecutor(len(SOURCES)) as ex:
        results = list(ex.map(lambda s: _compile(s, extra), SOURCES))
    objs = [o for o, _ in results]
    if verbose or resource_usage:
        for _, log in results:
            for line in log.splitlines():
                if "remark" in line or "error" in line:
                    print(line)
    tmp = LIB + ".tmp"
    r = subprocess.run([_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(resource_usage="--resource-usage" in sys.argv, verbose=True))
