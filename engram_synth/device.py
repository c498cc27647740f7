"""Fill device tensors with the seeded synthetic streams of ``engram_synth``.

Same element definition as the host generator (counter-mode SplitMix64,
Irwin-Hall(4), optional bf16 rounding); used for arrays too large to build on
the host.  Input generation only: no step of the Engram method lives here.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

from . import ih4_scale, stream_key

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libengram_synth.so")
SRC_PATH = os.path.join(_HERE, "csrc", "synth_fill.hip")

HIPCC_FLAGS = ["--offload-arch=gfx950", "-mcode-object-version=5", "-O3", "-fPIC", "-shared", "-std=c++17",
               "-ffp-contract=off",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose: bool = False) -> str:
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, SRC_PATH, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for synth_fill.hip:\n" + r.stderr)
    if verbose and r.stderr.strip():
        print(r.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(LIB_PATH)
        lib.synth_fill_ih4.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_int64,
                                       ctypes.c_float, ctypes.c_float, ctypes.c_int, ctypes.c_void_p]
        lib.synth_fill_ih4.restype = ctypes.c_int
        _lib = lib
    return _lib


def fill(tensor, seed: int, stream_id: int, sigma: float, bias: float = 0.0, base: int = 0) -> None:
    """Fill a contiguous float32/bfloat16 CUDA tensor with stream elements base.. ."""
    import torch

    if not tensor.is_cuda or not tensor.is_contiguous():
        raise ValueError("fill needs a contiguous device tensor")
    if tensor.dtype == torch.bfloat16:
        dt = 1
    elif tensor.dtype == torch.float32:
        dt = 0
    else:
        raise ValueError(f"unsupported dtype {tensor.dtype}")
    stream = torch.cuda.current_stream(tensor.device).cuda_stream
    rc = _load().synth_fill_ih4(ctypes.c_void_p(tensor.data_ptr()), tensor.numel(), stream_key(seed, stream_id),
                                base, float(ih4_scale(sigma)), float(bias), dt, ctypes.c_void_p(stream))
    if rc != 0:
        raise RuntimeError(f"synth_fill_ih4 failed with hipError {rc}")


def device_inputs(inp, device="cuda", hidden: bool = True) -> dict:
    """All inputs of one workload as device tensors: ids/remap copied from the
    host generator, real arrays filled on the device from their streams."""
    import numpy as np
    import torch

    w = inp.w
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    def gen(name, shape):
        t = torch.empty(shape, dtype=dt, device=device)
        stream_id, sigma, bias = inp.recipe(name)
        fill(t, w.seed, stream_id, sigma, bias)
        return t

    out = {
        "ids": torch.from_numpy(np.ascontiguousarray(inp.ids)).to(device),
        "remap": torch.from_numpy(inp.remap).to(device),
        "tables": gen("table", inp.table_shape()),
        "w_kv": gen("wkv", inp.wkv_shape()),
        "gamma_k": gen("gamma_k", (w.hc_mult, w.hidden)),
        "gamma_q": gen("gamma_q", (w.hc_mult, w.hidden)),
        "conv_w": gen("conv_w", (w.hc_mult, w.hidden, w.conv_kernel)),
    }
    if hidden:
        out["hidden"] = gen("hidden", inp.hidden_shape())
    return out


def storage_numpy(t):
    """A device tensor in the host generator's storage form (float32, or uint16 bf16 bits)."""
    import torch

    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    return t.numpy()
