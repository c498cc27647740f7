"""Engram conditional-memory forward pass on MI355X: Python binding of libengram.so.

Thin ctypes marshalling over the C ABI in include/engram.h.  Every step of the
forward pass runs in the library's HIP kernels; torch is used only to own
device memory and to name the stream.  The module raises ImportError if the
library is not built, and there is no fallback.

    cfg = EngramConfig.make(batch=4, seqlen=1024, ...)
    p = Params(remap=..., tables=..., w_kv=..., gamma_k=..., gamma_q=..., conv_w=...)
    out = forward(cfg, p, ids, hidden)            # [B][T][hc][d]
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

from ._build import DEBUG_LIB_PATH, LIB_PATH, build, source_hash  # noqa: F401

MAX_ORDERS = 8
MAX_HEADS = 64
F32, BF16 = 0, 1

STATUS = {0: "ok", -1: "invalid configuration or argument", -2: "workspace too small",
          -3: "HIP launch or API call failed", -4: "configuration not supported by the kernels"}

# every entry point the header declares, in its order
ENTRY_POINTS = ["engram_workspace_size", "engram_state_bytes_per_sequence", "engram_hash", "engram_hash_layers",
                "engram_gather", "engram_gather_host", "engram_project", "engram_gate_conv", "engram_forward",
                "engram_forward_noalloc", "engram_forward_gathered", "engram_backward_workspace_size", "engram_backward",
                "engram_backward_sparse", "engram_backward_saved_sparse",
                "engram_forward_train", "engram_backward_saved",
                "engram_forward_timed", "engram_forward_kernel_name", "engram_status_string"]


class EngramError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({status})")
        self.status = status


class EngramConfig(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("seqlen", ctypes.c_int32), ("vocab", ctypes.c_int32),
        ("n_orders", ctypes.c_int32), ("orders", ctypes.c_int32 * MAX_ORDERS),
        ("heads_per_order", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("hidden", ctypes.c_int32), ("hc_mult", ctypes.c_int32),
        ("conv_kernel", ctypes.c_int32), ("conv_dilation", ctypes.c_int32),
        ("pad_id", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("norm_eps", ctypes.c_float), ("gate_clamp", ctypes.c_float),
        ("multipliers", ctypes.c_int64 * MAX_ORDERS),
        ("primes", ctypes.c_int64 * MAX_HEADS),
    ]

    @classmethod
    def make(cls, *, batch: int, seqlen: int, vocab: int, orders: Sequence[int], heads_per_order: int,
             head_dim: int, hidden: int, hc_mult: int, multipliers: Sequence[int], primes: Sequence[int],
             conv_kernel: int = 4, conv_dilation: Optional[int] = None, pad_id: int = 0, dtype: str = "bf16",
             norm_eps: float = 1e-6, gate_clamp: float = 1e-6) -> "EngramConfig":
        c = cls()
        c.batch, c.seqlen, c.vocab = batch, seqlen, vocab
        if not 1 <= len(orders) <= MAX_ORDERS or len(primes) > MAX_HEADS or len(multipliers) > MAX_ORDERS:
            raise ValueError("too many orders, heads or multipliers")
        c.n_orders = len(orders)
        for i, o in enumerate(orders):
            c.orders[i] = int(o)
        c.heads_per_order, c.head_dim, c.hidden, c.hc_mult = heads_per_order, head_dim, hidden, hc_mult
        c.conv_kernel = conv_kernel
        c.conv_dilation = max(orders) if conv_dilation is None else conv_dilation
        c.pad_id = pad_id
        c.dtype = BF16 if dtype == "bf16" else F32
        c.norm_eps, c.gate_clamp = norm_eps, gate_clamp
        for i, m in enumerate(multipliers):
            c.multipliers[i] = int(m)
        for i, p in enumerate(primes):
            c.primes[i] = int(p)
        return c

    def with_shape(self, batch: int, seqlen: int) -> "EngramConfig":
        c = EngramConfig.from_buffer_copy(self)
        c.batch, c.seqlen = batch, seqlen
        return c

    @property
    def n_heads(self) -> int:
        return self.n_orders * self.heads_per_order

    @property
    def emb_dim(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def max_order(self) -> int:
        return self.orders[self.n_orders - 1]

    @property
    def ring_len(self) -> int:
        """Positions the value and gate rings of a state keep: the conv's history plus one."""
        return (self.conv_kernel - 1) * self.conv_dilation + 1


class _Params(ctypes.Structure):
    _fields_ = [("remap", ctypes.c_void_p), ("tables", ctypes.c_void_p), ("w_kv", ctypes.c_void_p),
                ("gamma_k", ctypes.c_void_p), ("gamma_q", ctypes.c_void_p), ("conv_w", ctypes.c_void_p)]


class _State(ctypes.Structure):
    _fields_ = [("tok_ring", ctypes.c_void_p), ("v_ring", ctypes.c_void_p), ("g_ring", ctypes.c_void_p),
                ("n_past", ctypes.c_void_p)]


_lib = None


def load(debug: bool = False):
    """The loaded library; ImportError if it has not been built.  debug=True:
    the ENGRAM_DEBUG build (libengram_debug.so), whose calls also check on the
    host that the raw token ids lie in [0, vocab)."""
    global _lib
    if debug:
        if "debug" not in _debug_lib:
            _debug_lib["debug"] = _open(DEBUG_LIB_PATH)
        return _debug_lib["debug"]
    if _lib is None:
        _lib = _open(LIB_PATH)
    return _lib


_debug_lib: dict = {}


def _open(path):
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    P, I = ctypes.c_void_p, ctypes.c_int
    cfgp = ctypes.POINTER(EngramConfig)
    prmp = ctypes.POINTER(_Params)
    stp = ctypes.POINTER(_State)
    lib.engram_workspace_size.argtypes = [cfgp]
    lib.engram_workspace_size.restype = ctypes.c_size_t
    lib.engram_state_bytes_per_sequence.argtypes = [cfgp]
    lib.engram_state_bytes_per_sequence.restype = ctypes.c_size_t
    lib.engram_hash.argtypes = [cfgp, prmp, P, stp, P, P]
    lib.engram_hash_layers.argtypes = [cfgp, prmp, P, stp, ctypes.POINTER(ctypes.c_int64), ctypes.c_int32, P, P]
    lib.engram_gather.argtypes = [cfgp, prmp, P, P, P]
    lib.engram_gather_host.argtypes = [cfgp, P, P, P, ctypes.c_int32]
    lib.engram_project.argtypes = [cfgp, prmp, P, P, P]
    lib.engram_gate_conv.argtypes = [cfgp, prmp, P, P, stp, P, P, P]
    lib.engram_forward.argtypes = [cfgp, prmp, P, P, stp, P, P, ctypes.c_size_t, P]
    lib.engram_forward_noalloc.argtypes = [cfgp, prmp, P, P, stp, P, P]
    lib.engram_forward_gathered.argtypes = [cfgp, prmp, P, P, P, stp, P, P, ctypes.c_size_t, P]
    lib.engram_backward_workspace_size.argtypes = [cfgp]
    lib.engram_backward_workspace_size.restype = ctypes.c_size_t
    lib.engram_backward.argtypes = [cfgp, prmp, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.engram_forward_train.argtypes = [cfgp, prmp, P, P, P, P, ctypes.c_size_t, P]
    lib.engram_backward_sparse.argtypes = [cfgp, prmp, P, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.engram_backward_saved_sparse.argtypes = [cfgp, prmp, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.engram_backward_saved.argtypes = [cfgp, prmp, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.engram_forward_timed.argtypes = [cfgp, prmp, P, P, stp, P, P, ctypes.c_size_t, P, P, ctypes.c_int32,
                                         ctypes.POINTER(ctypes.c_int32)]
    lib.engram_forward_kernel_name.argtypes = [cfgp, ctypes.c_int32, ctypes.c_int32]
    lib.engram_forward_kernel_name.restype = ctypes.c_char_p
    lib.engram_status_string.argtypes = [I]
    lib.engram_status_string.restype = ctypes.c_char_p
    for f in ("engram_hash", "engram_hash_layers", "engram_gather", "engram_gather_host", "engram_project",
              "engram_gate_conv", "engram_forward", "engram_forward_noalloc", "engram_forward_gathered", "engram_backward",
              "engram_forward_train", "engram_backward_saved", "engram_forward_timed", "engram_backward_sparse",
              "engram_backward_saved_sparse"):
        getattr(lib, f).restype = I
    return lib


# ------------------------------------------------------------------ marshalling
class MappedHost:
    """Pinned host memory mapped into the device (e.g. host-resident tables):
    `address` is the device-side address kernels use, from
    hipHostGetDevicePointer.  Allocate with alloc_mapped_host."""

    def __init__(self, address: int, host: int, nbytes: int):
        self.address, self.host, self.nbytes = address, host, nbytes

    def copy_from(self, t):
        """Copy a contiguous device tensor's bytes into the start of this buffer."""
        import torch

        n = t.numel() * t.element_size()
        if n > self.nbytes or not t.is_contiguous():
            raise ValueError("tensor does not fit or is not contiguous")
        torch.cuda.synchronize()
        if _hip().hipMemcpy(ctypes.c_void_p(self.host), ctypes.c_void_p(t.data_ptr()), ctypes.c_size_t(n), 4) != 0:
            raise RuntimeError("hipMemcpy failed")

    def free(self):
        if self.host:
            _hip().hipHostFree(ctypes.c_void_p(self.host))
            self.host = self.address = 0


_hip_rt = None


def _hip():
    """The HIP runtime already loaded by torch and by the library."""
    global _hip_rt
    if _hip_rt is None:
        _hip_rt = ctypes.CDLL("libamdhip64.so.7")
        _hip_rt.hipHostMalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t, ctypes.c_uint]
        _hip_rt.hipHostGetDevicePointer.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p, ctypes.c_uint]
        _hip_rt.hipHostFree.argtypes = [ctypes.c_void_p]
        _hip_rt.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    return _hip_rt


HOST_MAPPED, HOST_COHERENT, HOST_NONCOHERENT = 0x2, 0x40000000, 0x80000000


def alloc_mapped_host(nbytes: int, coherent: bool = False) -> MappedHost:
    """Pinned host memory, mapped into the current device.  Non-coherent (the
    default) lets the device cache what it reads, which read-only tables allow."""
    import torch

    torch.cuda.init()
    h = ctypes.c_void_p()
    flags = HOST_MAPPED | (HOST_COHERENT if coherent else HOST_NONCOHERENT)
    if _hip().hipHostMalloc(ctypes.byref(h), ctypes.c_size_t(nbytes), flags) != 0 or not h.value:
        raise MemoryError(f"hipHostMalloc of {nbytes} bytes failed")
    d = ctypes.c_void_p()
    if _hip().hipHostGetDevicePointer(ctypes.byref(d), h, 0) != 0:
        _hip().hipHostFree(h)
        raise RuntimeError("hipHostGetDevicePointer failed")
    return MappedHost(d.value, h.value, nbytes)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, MappedHost):
        return t.address
    if not t.is_cuda:
        raise ValueError("engram arguments must be device tensors")
    if not t.is_contiguous():
        raise ValueError("engram arguments must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _check(fn: str, rc: int):
    if rc != 0:
        raise EngramError(fn, rc)


class Params:
    """Device tensors of one Engram layer (see engram_params in include/engram.h)."""

    def __init__(self, *, tables, w_kv, gamma_k, gamma_q, conv_w, remap=None):
        self.remap, self.tables, self.w_kv = remap, tables, w_kv
        self.gamma_k, self.gamma_q, self.conv_w = gamma_k, gamma_q, conv_w
        self._c = _Params(_ptr(remap), _ptr(tables), _ptr(w_kv), _ptr(gamma_k), _ptr(gamma_q), _ptr(conv_w))


class State:
    """Decode state of `batch` sequences: token, value and gate rings plus n_past."""

    def __init__(self, cfg: EngramConfig, batch: int, device="cuda"):
        import torch

        dt = torch.bfloat16 if cfg.dtype == BF16 else torch.float32
        R = cfg.ring_len
        self.tok_ring = torch.zeros((batch, max(cfg.max_order - 1, 1)), dtype=torch.int32, device=device)
        self.v_ring = torch.zeros((batch, max(R, 1), cfg.hidden), dtype=dt, device=device)
        self.g_ring = torch.zeros((batch, max(R, 1), cfg.hc_mult), dtype=torch.float32, device=device)
        self.n_past = torch.zeros((batch,), dtype=torch.int64, device=device)
        self._c = _State(_ptr(self.tok_ring), _ptr(self.v_ring), _ptr(self.g_ring), _ptr(self.n_past))

    def clone(self) -> "State":
        s = State.__new__(State)
        s.tok_ring, s.v_ring = self.tok_ring.clone(), self.v_ring.clone()
        s.g_ring, s.n_past = self.g_ring.clone(), self.n_past.clone()
        s._c = _State(_ptr(s.tok_ring), _ptr(s.v_ring), _ptr(s.g_ring), _ptr(s.n_past))
        return s


def _real_dtype(cfg):
    import torch

    return torch.bfloat16 if cfg.dtype == BF16 else torch.float32


def workspace_size(cfg: EngramConfig) -> int:
    return load().engram_workspace_size(ctypes.byref(cfg))


def state_bytes_per_sequence(cfg: EngramConfig) -> int:
    return load().engram_state_bytes_per_sequence(ctypes.byref(cfg))


def engram_hash(cfg: EngramConfig, p: Params, ids, state: Optional[State] = None, out=None, stream=None):
    import torch

    if out is None:
        out = torch.empty((cfg.batch, cfg.seqlen, cfg.n_heads), dtype=torch.int32, device=ids.device)
    st = None if state is None else ctypes.byref(state._c)
    _check("engram_hash", load().engram_hash(ctypes.byref(cfg), ctypes.byref(p._c), _ptr(ids), st, _ptr(out),
                                             _stream(stream)))
    return out


def engram_hash_layers(cfg: EngramConfig, p: Params, ids, multipliers, state: Optional[State] = None, out=None,
                       stream=None):
    """Indices of several layers in one pass: `multipliers` is [L][<=8] ints
    (layer l's m_k); returns int32 [L][B][T][H]."""
    import torch

    L = len(multipliers)
    flat = (ctypes.c_int64 * (L * MAX_ORDERS))()
    for l, ms in enumerate(multipliers):
        for k, m in enumerate(ms):
            flat[l * MAX_ORDERS + k] = ctypes.c_int64(int(m)).value
    if out is None:
        out = torch.empty((L, cfg.batch, cfg.seqlen, cfg.n_heads), dtype=torch.int32, device=ids.device)
    st = None if state is None else ctypes.byref(state._c)
    _check("engram_hash_layers", load().engram_hash_layers(ctypes.byref(cfg), ctypes.byref(p._c), _ptr(ids), st, flat,
                                                           L, _ptr(out), _stream(stream)))
    return out


def engram_gather(cfg: EngramConfig, p: Params, idx, out=None, stream=None):
    import torch

    if out is None:
        out = torch.empty((cfg.batch, cfg.seqlen, cfg.emb_dim), dtype=_real_dtype(cfg), device=idx.device)
    _check("engram_gather", load().engram_gather(ctypes.byref(cfg), ctypes.byref(p._c), _ptr(idx), _ptr(out),
                                                 _stream(stream)))
    return out


def _host_ptr(t) -> int:
    """Address of host memory: a MappedHost buffer, a CPU tensor or a numpy array."""
    if isinstance(t, MappedHost):
        return t.host
    if hasattr(t, "__array_interface__"):
        return t.__array_interface__["data"][0]
    if t.is_cuda or not t.is_contiguous():
        raise ValueError("engram_gather_host takes contiguous host memory")
    return t.data_ptr()


def engram_gather_host(cfg: EngramConfig, tables, idx, out, n_threads: int = 0):
    """Row lookup on the host (tables in host memory): out[n][h] = tables row
    idx[n][h] of head h.  `idx` and `out` are host tensors (pinned, for the DMA
    copies around it); synchronous."""
    _check("engram_gather_host", load().engram_gather_host(ctypes.byref(cfg), _host_ptr(tables), _host_ptr(idx),
                                                           _host_ptr(out), n_threads))
    return out


def engram_project(cfg: EngramConfig, p: Params, e, out=None, stream=None):
    import torch

    if out is None:
        out = torch.empty((cfg.batch, cfg.seqlen, cfg.hc_mult + 1, cfg.hidden), dtype=_real_dtype(cfg),
                          device=e.device)
    _check("engram_project", load().engram_project(ctypes.byref(cfg), ctypes.byref(p._c), _ptr(e), _ptr(out),
                                                   _stream(stream)))
    return out


def engram_gate_conv(cfg: EngramConfig, p: Params, kv, hidden, state: Optional[State] = None, g_out=None, out=None,
                     stream=None):
    import torch

    if out is None:
        out = torch.empty((cfg.batch, cfg.seqlen, cfg.hc_mult, cfg.hidden), dtype=_real_dtype(cfg),
                          device=kv.device)
    if g_out is None:
        g_out = torch.empty((cfg.batch, cfg.seqlen, cfg.hc_mult), dtype=torch.float32, device=kv.device)
    st = None if state is None else ctypes.byref(state._c)
    _check("engram_gate_conv", load().engram_gate_conv(ctypes.byref(cfg), ctypes.byref(p._c), _ptr(kv),
                                                       _ptr(hidden), st, _ptr(g_out), _ptr(out), _stream(stream)))
    return out, g_out


def alloc_workspace(cfg: EngramConfig, device="cuda"):
    import torch

    n = workspace_size(cfg)
    if n == 0 and cfg.batch * cfg.seqlen > 0:
        raise EngramError("engram_workspace_size", -1)
    return torch.empty((max(n, 256),), dtype=torch.uint8, device=device)


def forward(cfg: EngramConfig, p: Params, ids, hidden, state: Optional[State] = None, out=None, workspace=None,
            stream=None, events=None):
    """Engram.forward: returns out [B][T][hc][d].  With `events` (a list of
    2*k hipEvent_t handles) the i-th kernel is bracketed by events[2i], [2i+1]."""
    import torch

    if out is None:
        out = torch.empty((cfg.batch, cfg.seqlen, cfg.hc_mult, cfg.hidden), dtype=_real_dtype(cfg),
                          device=ids.device)
    if workspace is None:
        workspace = alloc_workspace(cfg, ids.device)
    st = None if state is None else ctypes.byref(state._c)
    lib = load()
    if events is None:
        rc = lib.engram_forward(ctypes.byref(cfg), ctypes.byref(p._c), _ptr(ids), _ptr(hidden), st, _ptr(out),
                                _ptr(workspace), workspace.numel(), _stream(stream))
        _check("engram_forward", rc)
    else:
        forward_timed(cfg, p, ids, hidden, events, state=state, out=out, workspace=workspace, stream=stream)
    return out


def forward_timed(cfg: EngramConfig, p: Params, ids, hidden, events, state: Optional[State] = None, out=None,
                  workspace=None, stream=None):
    """engram_forward_timed: forward with the i-th kernel bracketed by
    events[2i], events[2i+1] (hipEvent_t handles).  Returns (out, number of
    kernels launched)."""
    import torch

    if out is None:
        out = torch.empty((cfg.batch, cfg.seqlen, cfg.hc_mult, cfg.hidden), dtype=_real_dtype(cfg),
                          device=ids.device)
    if workspace is None:
        workspace = alloc_workspace(cfg, ids.device)
    st = None if state is None else ctypes.byref(state._c)
    arr = (ctypes.c_void_p * max(len(events), 1))(*events)
    nk = ctypes.c_int32(0)
    rc = load().engram_forward_timed(ctypes.byref(cfg), ctypes.byref(p._c), _ptr(ids), _ptr(hidden), st, _ptr(out),
                                     _ptr(workspace), workspace.numel(), _stream(stream), arr, len(events),
                                     ctypes.byref(nk))
    _check("engram_forward_timed", rc)
    return out, nk.value


NOALLOC_MAX_BYTES = 64 << 20   # ENGRAM_NOALLOC_MAX_BYTES


def forward_noalloc(cfg: EngramConfig, p: Params, ids, hidden, state: Optional[State] = None, out=None, stream=None):
    """engram_forward_noalloc: Engram.forward on the library's own device array
    (no workspace; the library allocates nothing).  Returns out."""
    import torch

    if out is None:
        out = torch.empty((cfg.batch, cfg.seqlen, cfg.hc_mult, cfg.hidden), dtype=_real_dtype(cfg),
                          device=ids.device)
    st = None if state is None else ctypes.byref(state._c)
    rc = load().engram_forward_noalloc(ctypes.byref(cfg), ctypes.byref(p._c), _ptr(ids), _ptr(hidden), st, _ptr(out),
                                       _stream(stream))
    _check("engram_forward_noalloc", rc)
    return out


def forward_gathered(cfg: EngramConfig, p: Params, e, hidden, ids=None, state: Optional[State] = None, out=None,
                     workspace=None, stream=None):
    """Engram.forward on rows gathered beforehand (`e` [B][T][E] as written by
    engram_gather); `ids` only when a state is advanced.  Returns out."""
    import torch

    if out is None:
        out = torch.empty((cfg.batch, cfg.seqlen, cfg.hc_mult, cfg.hidden), dtype=_real_dtype(cfg), device=e.device)
    if workspace is None:
        workspace = alloc_workspace(cfg, e.device)
    st = None if state is None else ctypes.byref(state._c)
    rc = load().engram_forward_gathered(ctypes.byref(cfg), ctypes.byref(p._c), _ptr(ids), _ptr(e), _ptr(hidden), st,
                                        _ptr(out), _ptr(workspace), workspace.numel(), _stream(stream))
    _check("engram_forward_gathered", rc)
    return out


GRAD_NAMES = ("d_tables", "d_w_kv", "d_gamma_k", "d_gamma_q", "d_conv_w")


def backward_workspace_size(cfg: EngramConfig) -> int:
    return load().engram_backward_workspace_size(ctypes.byref(cfg))


def alloc_backward_workspace(cfg: EngramConfig, device="cuda"):
    import torch

    return torch.empty((max(backward_workspace_size(cfg), 256),), dtype=torch.uint8, device=device)


def _zero_grads(cfg: EngramConfig, dev, tables: bool = True):
    import torch

    E, d, hc = cfg.emb_dim, cfg.hidden, cfg.hc_mult
    rows = sum(int(cfg.primes[h]) for h in range(cfg.n_heads))
    shapes = {"d_tables": (rows, cfg.head_dim), "d_w_kv": ((hc + 1) * d, E), "d_gamma_k": (hc, d),
              "d_gamma_q": (hc, d), "d_conv_w": (hc, d, cfg.conv_kernel)}
    if not tables:
        del shapes["d_tables"]
    return {k: torch.zeros(v, dtype=torch.float32, device=dev) for k, v in shapes.items()}


def backward(cfg: EngramConfig, p: Params, ids, hidden, dy, grads=None, d_hidden=None, workspace=None, stream=None):
    """Gradients of Engram.forward for an upstream gradient dy.  `grads`: dict
    of float32 tensors named GRAD_NAMES, added to (allocated as zeros when
    None).  Returns (d_hidden, grads)."""
    import torch

    dev = ids.device
    if grads is None:
        grads = _zero_grads(cfg, dev)
    if d_hidden is None:
        d_hidden = torch.empty_like(hidden)
    if workspace is None:
        workspace = alloc_backward_workspace(cfg, dev)
    rc = load().engram_backward(ctypes.byref(cfg), ctypes.byref(p._c), _ptr(ids), _ptr(hidden), _ptr(dy),
                                _ptr(d_hidden), *[_ptr(grads[k]) for k in GRAD_NAMES], _ptr(workspace),
                                workspace.numel(), _stream(stream))
    _check("engram_backward", rc)
    return d_hidden, grads


SPARSE_GRAD_NAMES = ("d_w_kv", "d_gamma_k", "d_gamma_q", "d_conv_w")


def _sparse_outputs(cfg: EngramConfig, dev):
    import torch

    n = cfg.batch * cfg.seqlen * cfg.n_heads
    return {"row_index": torch.empty((n,), dtype=torch.int64, device=dev),
            "d_rows": torch.empty((n, cfg.head_dim), dtype=torch.float32, device=dev),
            "n_rows": torch.empty((1,), dtype=torch.int64, device=dev)}


def backward_sparse(cfg: EngramConfig, p: Params, ids, hidden, dy, grads=None, rows=None, d_hidden=None,
                    workspace=None, stream=None):
    """Gradients with the table gradient row-sparse: returns (d_hidden, grads,
    rows), rows = {"row_index", "d_rows", "n_rows"} (the first n_rows entries
    valid); grads holds the dense parameter gradients (added to)."""
    import torch

    dev = ids.device
    if grads is None:
        grads = {k: v for k, v in _zero_grads(cfg, dev, tables=False).items()}
    if rows is None:
        rows = _sparse_outputs(cfg, dev)
    if d_hidden is None:
        d_hidden = torch.empty_like(hidden)
    if workspace is None:
        workspace = alloc_backward_workspace(cfg, dev)
    rc = load().engram_backward_sparse(ctypes.byref(cfg), ctypes.byref(p._c), _ptr(ids), _ptr(hidden), _ptr(dy),
                                       _ptr(d_hidden), _ptr(rows["row_index"]), _ptr(rows["d_rows"]),
                                       _ptr(rows["n_rows"]), *[_ptr(grads[k]) for k in SPARSE_GRAD_NAMES],
                                       _ptr(workspace), workspace.numel(), _stream(stream))
    _check("engram_backward_sparse", rc)
    return d_hidden, grads, rows


def backward_saved_sparse(cfg: EngramConfig, p: Params, hidden, dy, workspace, grads=None, rows=None, d_hidden=None,
                          stream=None):
    """backward_sparse on the quantities forward_train kept in `workspace`."""
    import torch

    dev = hidden.device
    if grads is None:
        grads = {k: v for k, v in _zero_grads(cfg, dev, tables=False).items()}
    if rows is None:
        rows = _sparse_outputs(cfg, dev)
    if d_hidden is None:
        d_hidden = torch.empty_like(hidden)
    rc = load().engram_backward_saved_sparse(ctypes.byref(cfg), ctypes.byref(p._c), _ptr(hidden), _ptr(dy),
                                             _ptr(d_hidden), _ptr(rows["row_index"]), _ptr(rows["d_rows"]),
                                             _ptr(rows["n_rows"]), *[_ptr(grads[k]) for k in SPARSE_GRAD_NAMES],
                                             _ptr(workspace), workspace.numel(), _stream(stream))
    _check("engram_backward_saved_sparse", rc)
    return d_hidden, grads, rows


def forward_train(cfg: EngramConfig, p: Params, ids, hidden, workspace, out=None, stream=None):
    """Forward of a training step; `workspace` (alloc_backward_workspace) keeps
    what backward_saved needs.  Returns out [B][T][hc][d]."""
    import torch

    if out is None:
        out = torch.empty_like(hidden)
    rc = load().engram_forward_train(ctypes.byref(cfg), ctypes.byref(p._c), _ptr(ids), _ptr(hidden), _ptr(out),
                                     _ptr(workspace), workspace.numel(), _stream(stream))
    _check("engram_forward_train", rc)
    return out


def backward_saved(cfg: EngramConfig, p: Params, hidden, dy, workspace, grads=None, d_hidden=None, stream=None):
    """backward on the quantities forward_train kept in `workspace`.  Returns (d_hidden, grads)."""
    import torch

    if grads is None:
        grads = _zero_grads(cfg, hidden.device)
    if d_hidden is None:
        d_hidden = torch.empty_like(hidden)
    rc = load().engram_backward_saved(ctypes.byref(cfg), ctypes.byref(p._c), _ptr(hidden), _ptr(dy), _ptr(d_hidden),
                                      *[_ptr(grads[k]) for k in GRAD_NAMES], _ptr(workspace), workspace.numel(),
                                      _stream(stream))
    _check("engram_backward_saved", rc)
    return d_hidden, grads


def kernel_names(cfg: EngramConfig, with_state: bool = False):
    """Names of the kernels engram_forward launches for cfg, in launch order."""
    lib = load()
    names = []
    while True:
        nm = lib.engram_forward_kernel_name(ctypes.byref(cfg), int(with_state), len(names))
        if nm is None:
            break
        names.append(nm.decode())
    return names
