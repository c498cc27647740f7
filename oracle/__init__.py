"""ctypes wrapper around the Engram forward oracle (engram_oracle.c).

TEST INFRASTRUCTURE ONLY: the plain, slow, double-precision CPU definition of
the forward pass.  Only the tests, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg use it; the product library never does.

Parity pins (what fixes this oracle to the pages rather than to itself) live
in tests/test_oracle_pins.py.  Functions without a page-backed pin: the
choice of multipliers, primes, RMSNorm epsilon and the multiplier/offset
pairing are readings fixed by this oracle's header ("parity unpinned" against
the pages for those constants; the arithmetic that uses them is pinned).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC_PATH = os.path.join(_HERE, "engram_oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")

MAX_ORDERS = 8
MAX_HEADS = 64


def build() -> str:
    tmp = LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-Wall", "-Wextra", "-Wno-unused-parameter",
           SRC_PATH, "-o", tmp, "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("gcc failed for the oracle:\n" + r.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


class OrcConfig(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("seqlen", ctypes.c_int32),
        ("n_orders", ctypes.c_int32), ("orders", ctypes.c_int32 * MAX_ORDERS),
        ("heads_per_order", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("hidden", ctypes.c_int32), ("hc_mult", ctypes.c_int32),
        ("conv_kernel", ctypes.c_int32), ("conv_dilation", ctypes.c_int32),
        ("pad_id", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("norm_eps", ctypes.c_double), ("gate_clamp", ctypes.c_double),
        ("multipliers", ctypes.c_int64 * MAX_ORDERS),
        ("primes", ctypes.c_int64 * MAX_HEADS),
    ]


class OrcRows(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("keys", ctypes.c_void_p), ("n", ctypes.c_int64)]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        cp = ctypes.POINTER(OrcConfig)
        rp = ctypes.POINTER(OrcRows)
        lib.orc_shift.argtypes = [cp, P, P, ctypes.c_int, P]
        lib.orc_hash.argtypes = [cp, P, ctypes.c_int32, P, P, P]
        lib.orc_gather.argtypes = [cp, rp, P, ctypes.c_int64, P]
        lib.orc_project.argtypes = [cp, P, P, ctypes.c_int64, P]
        lib.orc_gate.argtypes = [cp, P, P, P, P, ctypes.c_int64, P, P]
        lib.orc_conv.argtypes = [cp, P, P, P, P]
        lib.orc_forward.argtypes = [cp, P, ctypes.c_int32, P, rp, P, P, P, P, P, P]
        lib.orc_forward_at.argtypes = [cp, P, ctypes.c_int32, P, rp, P, P, P, P, rp, ctypes.c_int64, P, P]
        lib.orc_backward.argtypes = [cp, P, ctypes.c_int32, P, rp, P, P, P, P, P, P, P, P, P, P, P, P]
        lib.orc_backward_at.argtypes = [cp, P, ctypes.c_int32, P, rp, P, P, P, P, rp, rp, ctypes.c_int64, P, P, P,
                                        P, P, P]
        for f in ("orc_shift", "orc_hash", "orc_gather", "orc_project", "orc_gate", "orc_conv", "orc_forward",
                  "orc_forward_at", "orc_backward", "orc_backward_at"):
            getattr(lib, f).restype = ctypes.c_int
        _lib = lib
    return _lib


class OracleError(RuntimeError):
    pass


def _ok(rc: int, what: str):
    if rc != 0:
        raise OracleError(f"{what} returned {rc}")


def _p(a: Optional[np.ndarray]):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


class Oracle:
    """One forward-pass configuration.  Real arrays are passed in storage form:
    float32 (dtype 'f32') or uint16 bfloat16 bits (dtype 'bf16')."""

    def __init__(self, *, batch: int, seqlen: int, orders: Sequence[int], heads_per_order: int, head_dim: int,
                 hidden: int, hc_mult: int, multipliers: Sequence[int], primes: Sequence[int], pad_id: int = 0,
                 conv_kernel: int = 4, conv_dilation: Optional[int] = None, dtype: str = "f32",
                 norm_eps: float = 1e-6, gate_clamp: float = 1e-6):
        c = OrcConfig()
        c.batch, c.seqlen = batch, seqlen
        if not 1 <= len(orders) <= MAX_ORDERS:
            raise ValueError("orders")
        c.n_orders = len(orders)
        for i, o in enumerate(orders):
            c.orders[i] = o
        c.heads_per_order, c.head_dim, c.hidden, c.hc_mult = heads_per_order, head_dim, hidden, hc_mult
        c.conv_kernel = conv_kernel
        c.conv_dilation = max(orders) if conv_dilation is None else conv_dilation
        c.pad_id = pad_id
        c.dtype = 0 if dtype == "f32" else 1
        c.norm_eps, c.gate_clamp = norm_eps, gate_clamp
        mults = [int(m) for m in multipliers]
        if len(mults) < max(orders):
            raise ValueError("need one multiplier per offset below the largest order")
        for i, m in enumerate(mults[:MAX_ORDERS]):
            c.multipliers[i] = m
        if len(primes) != len(orders) * heads_per_order:
            raise ValueError("need one prime per head")
        for i, p in enumerate(primes):
            c.primes[i] = int(p)
        self.cfg = c
        self.dtype = dtype
        self.store = np.float32 if dtype == "f32" else np.uint16
        self.n_heads = len(orders) * heads_per_order
        self.emb_dim = self.n_heads * head_dim
        self.max_order = max(orders)

    @classmethod
    def from_workload(cls, w, inputs, **over):
        kw = dict(batch=w.batch, seqlen=w.seqlen, orders=w.orders, heads_per_order=w.heads_per_order,
                  head_dim=w.head_dim, hidden=w.hidden, hc_mult=w.hc_mult, multipliers=inputs.multipliers,
                  primes=inputs.primes, pad_id=w.pad_id, conv_kernel=w.conv_kernel, conv_dilation=w.conv_dilation,
                  dtype=w.dtype, norm_eps=w.norm_eps, gate_clamp=w.gate_clamp)
        kw.update(over)
        return cls(**kw)

    def with_shape(self, batch: int, seqlen: int) -> "Oracle":
        o = Oracle.__new__(Oracle)
        o.__dict__.update(self.__dict__)
        c = OrcConfig.from_buffer_copy(self.cfg)
        c.batch, c.seqlen = batch, seqlen
        o.cfg = c
        return o

    @property
    def B(self):
        return self.cfg.batch

    @property
    def T(self):
        return self.cfg.seqlen

    # ---- steps
    def shift(self, x: np.ndarray, k: int, hist: Optional[np.ndarray] = None) -> np.ndarray:
        x = _c(x, np.int32)
        h = None if hist is None else _c(hist, np.int32)
        out = np.empty((self.B, self.T), np.int32)
        _ok(_load().orc_shift(ctypes.byref(self.cfg), _p(x), _p(h), k, _p(out)), "orc_shift")
        return out

    def hash(self, ids: np.ndarray, remap: Optional[np.ndarray] = None, hist: Optional[np.ndarray] = None):
        ids = _c(ids, np.int32)
        rm = None if remap is None else _c(remap, np.int32)
        h = None if hist is None else _c(hist, np.int32)
        out = np.empty((self.B, self.T, self.n_heads), np.int64)
        _ok(_load().orc_hash(ctypes.byref(self.cfg), _p(rm), 0 if rm is None else len(rm), _p(ids), _p(h),
                             _p(out)), "orc_hash")
        return out

    @staticmethod
    def _rows(data: np.ndarray, keys: Optional[np.ndarray]):
        r = OrcRows()
        r.data = data.ctypes.data
        r.keys = None if keys is None else keys.ctypes.data
        r.n = data.shape[0] if keys is None else len(keys)
        return r

    def gather(self, table: np.ndarray, idx: np.ndarray, keys: Optional[np.ndarray] = None) -> np.ndarray:
        table = _c(table, self.store)
        k = None if keys is None else _c(keys, np.int64)
        idx = _c(idx, np.int64)
        n = idx.size // self.n_heads
        out = np.empty((n, self.emb_dim), self.store)
        rows = self._rows(table, k)
        _ok(_load().orc_gather(ctypes.byref(self.cfg), ctypes.byref(rows), _p(idx), n, _p(out)), "orc_gather")
        return out

    def project(self, w_kv: np.ndarray, e: np.ndarray) -> np.ndarray:
        w_kv, e = _c(w_kv, self.store), _c(e, self.store)
        n = e.size // self.emb_dim
        c = self.cfg
        out = np.empty((n, c.hc_mult + 1, c.hidden), np.float64)
        _ok(_load().orc_project(ctypes.byref(c), _p(w_kv), _p(e), n, _p(out)), "orc_project")
        return out

    def gate(self, gamma_k, gamma_q, kv: np.ndarray, hidden: np.ndarray, want_score: bool = False):
        c = self.cfg
        gk, gq, hid = _c(gamma_k, self.store), _c(gamma_q, self.store), _c(hidden, self.store)
        kv = _c(kv, np.float64)
        n = kv.size // ((c.hc_mult + 1) * c.hidden)
        g = np.empty((n, c.hc_mult), np.float64)
        s = np.empty((n, c.hc_mult), np.float64) if want_score else None
        _ok(_load().orc_gate(ctypes.byref(c), _p(gk), _p(gq), _p(kv), _p(hid), n, _p(s), _p(g)), "orc_gate")
        return (g, s) if want_score else g

    def conv(self, conv_w, kv: np.ndarray, g: np.ndarray) -> np.ndarray:
        c = self.cfg
        w = _c(conv_w, self.store)
        kv, g = _c(kv, np.float64), _c(g, np.float64)
        out = np.empty((c.batch, c.seqlen, c.hc_mult, c.hidden), np.float64)
        _ok(_load().orc_conv(ctypes.byref(c), _p(w), _p(kv), _p(g), _p(out)), "orc_conv")
        return out

    def forward(self, ids, remap, table, w_kv, gamma_k, gamma_q, conv_w, hidden) -> np.ndarray:
        c = self.cfg
        ids, rm = _c(ids, np.int32), _c(remap, np.int32)
        table = _c(table, self.store)
        args = [_c(a, self.store) for a in (w_kv, gamma_k, gamma_q, conv_w, hidden)]
        out = np.empty((c.batch, c.seqlen, c.hc_mult, c.hidden), np.float64)
        rows = self._rows(table, None)
        _ok(_load().orc_forward(ctypes.byref(c), _p(rm), len(rm), _p(ids), ctypes.byref(rows),
                                *[_p(a) for a in args], _p(out)), "orc_forward")
        return out

    def forward_at(self, ids, remap, table, w_kv, gamma_k, gamma_q, conv_w, hidden, positions,
                   table_keys=None, hidden_keys=None) -> np.ndarray:
        """Outputs at flat positions b*T+t; table/hidden may be sparse (rows + ascending keys)."""
        c = self.cfg
        ids, rm = _c(ids, np.int32), _c(remap, np.int32)
        table = _c(table, self.store)
        hidden = _c(hidden, self.store).reshape(-1, c.hc_mult * c.hidden)
        tk = None if table_keys is None else _c(table_keys, np.int64)
        hk = None if hidden_keys is None else _c(hidden_keys, np.int64)
        args = [_c(a, self.store) for a in (w_kv, gamma_k, gamma_q, conv_w)]
        pos = _c(positions, np.int64)
        out = np.empty((len(pos), c.hc_mult, c.hidden), np.float64)
        trows, hrows = self._rows(table, tk), self._rows(hidden, hk)
        _ok(_load().orc_forward_at(ctypes.byref(c), _p(rm), len(rm), _p(ids), ctypes.byref(trows), *[_p(a) for a in args],
                                   ctypes.byref(hrows), len(pos), _p(pos), _p(out)), "orc_forward_at")
        return out


    def backward(self, ids, remap, table, w_kv, gamma_k, gamma_q, conv_w, hidden, dy) -> dict:
        """Gradients of the module (orc_backward) for an upstream gradient dy
        [B][T][hc][d]: dict of float64 arrays d_table [rows][Dh], d_w_kv,
        d_gamma_k, d_gamma_q, d_conv_w, d_hidden (shapes of the inputs)."""
        c = self.cfg
        ids, rm = _c(ids, np.int32), _c(remap, np.int32)
        table = _c(table, self.store)
        args = [_c(a, self.store) for a in (w_kv, gamma_k, gamma_q, conv_w, hidden)]
        dy = _c(dy, np.float64)
        H, d, hc = self.n_heads, c.hidden, c.hc_mult
        E = H * c.head_dim
        rows = int(sum(int(c.primes[h]) for h in range(H)))
        out = {"d_table": np.empty((rows, c.head_dim)), "d_w_kv": np.empty(((hc + 1) * d, E)),
               "d_gamma_k": np.empty((hc, d)), "d_gamma_q": np.empty((hc, d)),
               "d_conv_w": np.empty((hc, d, c.conv_kernel)), "d_hidden": np.empty((c.batch, c.seqlen, hc, d))}
        trows = self._rows(table, None)
        _ok(_load().orc_backward(ctypes.byref(c), _p(rm), len(rm), _p(ids), ctypes.byref(trows),
                                 *[_p(a) for a in args], _p(dy),
                                 *[_p(out[k]) for k in ("d_table", "d_w_kv", "d_gamma_k", "d_gamma_q", "d_conv_w",
                                                       "d_hidden")]), "orc_backward")
        return out

    def backward_at(self, ids, remap, table, w_kv, gamma_k, gamma_q, conv_w, hidden, dy, positions,
                    table_keys=None, hidden_keys=None, dy_keys=None, want_de: bool = True, want_dkv: bool = False,
                    want_dgamma: bool = False):
        """orc_backward_at: (d_hidden [P][hc][d], de [P][E] or None) at flat positions;
        with want_dkv also dkv [P][(hc+1)][d] (the keys' and value's gradient at
        each position), with want_dgamma also (d_gamma_k, d_gamma_q) [hc][d], the
        sums of the positions' terms.  table, hidden and dy may be sparse (rows +
        ascending keys); hidden and dy rows are keyed by flat position, [hc][d]
        each, in storage form."""
        c = self.cfg
        ids, rm = _c(ids, np.int32), _c(remap, np.int32)
        table = _c(table, self.store)
        hidden = _c(hidden, self.store).reshape(-1, c.hc_mult * c.hidden)
        dy = _c(dy, self.store).reshape(-1, c.hc_mult * c.hidden)
        tk = None if table_keys is None else _c(table_keys, np.int64)
        hk = None if hidden_keys is None else _c(hidden_keys, np.int64)
        yk = None if dy_keys is None else _c(dy_keys, np.int64)
        args = [_c(a, self.store) for a in (w_kv, gamma_k, gamma_q, conv_w)]
        pos = _c(positions, np.int64)
        dh = np.empty((len(pos), c.hc_mult, c.hidden), np.float64)
        de = np.empty((len(pos), self.emb_dim), np.float64) if want_de else None
        dkv = np.empty((len(pos), c.hc_mult + 1, c.hidden), np.float64) if want_dkv else None
        dgk = np.zeros((c.hc_mult, c.hidden), np.float64) if want_dgamma else None
        dgq = np.zeros((c.hc_mult, c.hidden), np.float64) if want_dgamma else None
        trows, hrows, yrows = self._rows(table, tk), self._rows(hidden, hk), self._rows(dy, yk)
        _ok(_load().orc_backward_at(ctypes.byref(c), _p(rm), len(rm), _p(ids), ctypes.byref(trows),
                                    *[_p(a) for a in args], ctypes.byref(hrows), ctypes.byref(yrows), len(pos),
                                    _p(pos), _p(dh), _p(de), _p(dkv), _p(dgk), _p(dgq)), "orc_backward_at")
        out = (dh, de)
        if want_dkv:
            out = out + (dkv,)
        if want_dgamma:
            out = out + (dgk, dgq)
        return out


def needed_positions(T: int, positions: np.ndarray, conv_kernel: int, dilation: int) -> np.ndarray:
    """Sorted flat positions whose e/K/V/g the outputs at `positions` read through the causal conv."""
    pos = np.asarray(positions, dtype=np.int64)
    b, t = pos // T, pos % T
    out = []
    for j in range(conv_kernel):
        tau = t - (conv_kernel - 1 - j) * dilation
        ok = tau >= 0
        out.append(b[ok] * T + tau[ok])
    return np.unique(np.concatenate(out))
