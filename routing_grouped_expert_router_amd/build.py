"""Build libmoe.so (the HIP kernels and their C ABI) for gfx950, in-tree.

    python -m routing_grouped_expert_router_amd.build

Every call recompiles. Objects go to ``_build/`` next to this file; the
shared library lands in this package directory, where the binding loads it.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys
from typing import Dict, List

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmoe.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed binary32 VALU ops are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def sources() -> List[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


RESOURCE_REMARK = "-Rpass-analysis=kernel-resource-usage"


def resource_report(src: str) -> str:
    """Path of the per-kernel resource summary (registers, scratch, spills,
    LDS) that the last build wrote for `src`."""
    return os.path.join(BUILD, os.path.basename(src)[:-4] + ".resources.txt")


def parse_resources(text: str) -> Dict[str, Dict[str, str]]:
    """{kernel: {field: value}} from the compiler's kernel-resource remarks."""
    out: Dict[str, Dict[str, str]] = {}
    cur = None
    for line in text.splitlines():
        m = re.search(r"remark:\s+(.*?) \[-Rpass-analysis=kernel-resource-usage\]", line)
        if not m:
            continue
        key, _, val = m.group(1).strip().partition(": ")
        if key == "Function Name":
            cur = out.setdefault(val.strip(), {})
        elif cur is not None:
            cur[key] = val.strip()
    return out


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = [_hipcc(), *HIPCC_FLAGS, RESOURCE_REMARK, "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{err}")
    with open(resource_report(src), "w") as f:
        f.write("\n".join(l for l in err.splitlines() if "kernel-resource-usage" in l) + "\n")
    rest = "\n".join(l for l in err.splitlines() if "kernel-resource-usage" not in l and "remark" not in l)
    if rest.strip() and verbose:
        print(rest)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking libmoe.so failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
