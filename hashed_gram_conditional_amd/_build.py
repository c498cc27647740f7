"""Build step of the Engram HIP library: hipcc for gfx950 into an in-tree .so."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_PATH = os.path.join(PKG, "libengram.so")
SOURCES = ["engram_abi.hip", "hash_gather.hip", "gemm.hip", "gemm_tn.hip", "gate_conv.hip", "backward.hip"]
HEADERS = ["engram_internal.h", "gemm_common.h", os.path.join("..", "..", "include", "engram.h")]

HIPCC_FLAGS = ["--offload-arch=gfx950", "-mcode-object-version=5", "-O3", "-fPIC", "-shared", "-std=c++20", "-Wall",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-I" + os.path.join(ROOT, "include")]


# the sources the forward kernels are built from (the gradients' kernels are not among them)
FORWARD_SOURCES = [f for f in SOURCES if f not in ("backward.hip", "gemm_tn.hip")]


def source_hash() -> str:
    """sha256 over the forward kernels' sources and headers: identifies the
    build that measured HBM traffic per forward kernel describes."""
    import hashlib

    h = hashlib.sha256()
    for f in sorted(FORWARD_SOURCES + HEADERS):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def hipcc() -> str:
    return os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")


def build(verbose: bool = False) -> str:
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for libengram.so:\n" + r.stderr[-20000:])
    if verbose:
        print(" ".join(cmd))
        noise = "is not a recognized feature for this target"
        err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
        if err.strip():
            print(err)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
