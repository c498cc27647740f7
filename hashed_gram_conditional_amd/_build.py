"""Build step of the Engram HIP library: hipcc for gfx950 into in-tree .so files.

libengram.so is the library; libengram_debug.so is the same library built
with ENGRAM_DEBUG, whose calls also check on the host that every raw token id
lies in [0, vocab) and return ENGRAM_EINVAL otherwise (the release build
hashes such an id as pad_id).  Each source is compiled to an object in its own
hipcc process, in parallel; the two libraries share every object but the ABI's.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_PATH = os.path.join(PKG, "libengram.so")
DEBUG_LIB_PATH = os.path.join(PKG, "libengram_debug.so")
OBJ_DIR = os.path.join(ROOT, "_build", "obj")
SOURCES = ["engram_abi.hip", "hash_gather.hip", "gemm.hip", "gemm_tn.hip", "gate_conv.hip", "backward.hip",
           "sparse_grad.hip"]
HEADERS = ["engram_internal.h", "gemm_common.h", os.path.join("..", "..", "include", "engram.h")]

HIPCC_FLAGS = ["--offload-arch=gfx950", "-mcode-object-version=5", "-O3", "-fPIC", "-std=c++20", "-Wall",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-I" + os.path.join(ROOT, "include")]


# the sources the forward kernels are built from (the gradients' kernels are not among them)
FORWARD_SOURCES = [f for f in SOURCES if f not in ("backward.hip", "gemm_tn.hip", "sparse_grad.hip")]


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


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + r.stderr[-20000:])
    return r


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    compiles = [(s, [], os.path.join(OBJ_DIR, s.replace(".hip", ".o"))) for s in SOURCES]
    compiles.append(("engram_abi.hip", ["-DENGRAM_DEBUG"], os.path.join(OBJ_DIR, "engram_abi_debug.o")))
    with concurrent.futures.ThreadPoolExecutor(max(1, min(jobs, len(compiles)))) as ex:
        outs = list(ex.map(lambda c: _run([hipcc(), *HIPCC_FLAGS, *c[1], "-c", os.path.join(CSRC, c[0]),
                                          "-o", c[2]]), compiles))
    if verbose:
        noise = "is not a recognized feature for this target"
        for r in outs:
            err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
            if err.strip():
                print(err)
    objs = {s: o for s, _, o in compiles[:len(SOURCES)]}
    for lib, abi in ((LIB_PATH, objs["engram_abi.hip"]), (DEBUG_LIB_PATH, compiles[-1][2])):
        tmp = lib + ".tmp"
        _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", abi,
              *[objs[s] for s in SOURCES if s != "engram_abi.hip"], "-o", tmp])
        os.replace(tmp, lib)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
