"""Build libpa.so (HIP, gfx950) in place next to this file.

Usage: ``python -m paged_kv_cache_192_amd.build [--verbose]``.  Each source is
compiled to an object in ``_build/`` (in parallel), then linked.  The
library is always rebuilt when this runs.
"""
from __future__ import annotations

import concurrent.futures
import glob
import re
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build", "libpa")
LIB = os.path.join(HERE, "libpa.so")
ARCH = os.environ.get("PA_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "--offload-arch=%s" % ARCH,
    "-I", INCLUDE, "-I", CSRC,
    # Packed fp32 instructions are kept out of every kernel (the compiler
    # would otherwise form v_pk_* fp32 ops from plain float code).
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: the softmax rescale multiplies them with
    # ordinary vector instructions, which cannot read AGPRs.
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def _scratch_users(remarks: str) -> list:
    """Kernels that spill vector registers or use scratch memory, from the
    compiler's kernel-resource-usage remarks."""
    bad, cur = [], None
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            continue
        m = re.search(r"(VGPRs Spill|ScratchSize \[bytes/lane\]): (\d+)", line)
        if m and cur and int(m.group(2)) > 0:
            bad.append("%s: %s %s" % (cur, m.group(1), m.group(2)))
    return bad


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC] + COMMON + ["-c", src, "-o", obj]
    device = src.endswith(".hip")
    if device:
        cmd += ["-Rpass-analysis=kernel-resource-usage"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in line and "is not a recognized feature" not in line)
    if res.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s" % (" ".join(cmd), out))
    if verbose and out.strip():
        print(out)
    # every kernel keeps its working set in registers: a spill or a stack
    # array in scratch memory would cost far more than it saves
    bad = _scratch_users(out) if device else []
    if bad:
        raise RuntimeError("kernels in %s use scratch memory:\n  %s" % (os.path.basename(src), "\n  ".join(bad)))
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=%s" % ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed: %s\n%s" % (" ".join(cmd), res.stdout + res.stderr))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
