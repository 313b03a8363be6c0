"""Build libspa2.so (gfx950) in-tree with hipcc.

Every .hip kernel file and the C ABI layer are compiled to objects in parallel and
linked into block_sparse_attention_spa2_amd/libspa2.so. Always rebuilds.

Usage: python -m block_sparse_attention_spa2_amd.build
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libspa2.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    # no packed fp32 ALU ops in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
SOURCES = ["mask.hip", "fwd.hip", "bwd.hip", "diag.hip", "api.cpp"]


# the compiler's per-kernel resource report (registers, spills, LDS), read by _spills
REMARKS = ["-Rpass-analysis=kernel-resource-usage"]


def _spills(text: str) -> list:
    """(kernel, spilled VGPRs) for every kernel of a resource report that spills."""
    found, name = [], None
    for line in text.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"remark:\s+VGPRs Spill: (\d+)", line)
        if m and name is not None and int(m.group(1)) > 0:
            found.append((name, int(m.group(1))))
    return found


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src + ".o")
    cmd = [HIPCC, *FLAGS, *REMARKS, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    text = r.stdout + r.stderr
    out = "\n".join(x for x in text.splitlines()
                    if "packed-fp32-ops" not in x and "remark:" not in x)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    # The bf16 and mask kernels are sized to keep every value in registers (the forward's
    # launch bounds ask for three workgroups per CU, at most 168 registers): a spill to
    # scratch memory would cost far more than it saves, so it is a build error. The fp32
    # attention kernels (first template argument float, mangled "kernelIf") are the
    # precision path and do spill at D = 128.
    spills = [(n, c) for n, c in _spills(text) if "kernelIf" not in n]
    if spills:
        raise RuntimeError(f"register spills in {src}: " +
                           ", ".join(f"{n} ({c} VGPRs)" for n, c in spills))
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
