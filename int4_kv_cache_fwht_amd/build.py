"""Builds ``libkv4.so`` (HIP kernels for gfx950 + the C ABI) in-tree with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libkv4.so")
BUILD_DIR = os.path.join(PKG, "_build")

ARCH = "gfx950"
KERNEL_SOURCES = ["kv4_append.hip", "kv4_decode.hip", "kv4_mq.hip", "kv4_probe.hip"]
# -ffp-contract=off: the append's binary32 steps must not fuse into FMAs.
# -packed-fp32-ops off: no packed fp32 VALU instructions in any kernel.
HIPFLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found")
    return p


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "is not a recognized feature" not in l)
    if r.returncode != 0:
        sys.stderr.write(out + "\n")
        raise RuntimeError("command failed: " + " ".join(cmd))
    return out


def build(verbose: bool = False) -> str:
    """Compile every source; always recompiles.  Returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    hipcc = _hipcc()
    inc = ["-I", INCLUDE, "-I", CSRC]
    kobjs = []
    for src in KERNEL_SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        # the compiler's per-kernel resource report (registers, scratch, occupancy) is kept beside
        # the object; a CPU test checks that no kernel uses scratch memory
        out = _run([hipcc, "--offload-arch=" + ARCH, *HIPFLAGS, *inc, "-Rpass-analysis=kernel-resource-usage", "-c",
                    os.path.join(CSRC, src), "-o", obj])
        with open(os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".resources.txt"), "w") as f:
            f.write(out)
        kobjs.append(obj)
    hobj = os.path.join(BUILD_DIR, "kv4_host.o")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    _run([hipcc, "-O2", "-std=c++17", "-fPIC", "-Wall", *inc, "-I", os.path.join(rocm, "include"), "-x", "c++",
          "-D__HIP_PLATFORM_AMD__", "-c", os.path.join(CSRC, "kv4_host.cpp"), "-o", hobj])
    tmp = LIB + ".tmp%d" % os.getpid()
    _run([hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC", *kobjs, hobj, "-o", tmp])
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
