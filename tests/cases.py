"""Shared test cases: one workload's seeded inputs, its device tensors and the
oracle evaluated at chosen positions (rows and hidden states regenerated on
the host only where those positions read them)."""
from __future__ import annotations

import concurrent.futures
import functools
import multiprocessing
import os

import numpy as np

import engram_synth as S
import oracle as orc


def normwise(x, ref) -> float:
    """max |x - ref| / max |ref| (the tolerance measure of the parity tests)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.abs(ref).max()
    return float(np.abs(x - ref).max() / (den if den > 0 else 1.0))


TOL = {"f32": 1e-5, "bf16": 2e-2}


def oracle_workers() -> int:
    """Worker processes for the oracle: the host's cores, at most 16."""
    return max(1, min(16, os.cpu_count() or 1))


_WORKER_CASES: dict = {}


def _worker_case(name, over):
    key = (name, repr(over))
    if key not in _WORKER_CASES:
        _WORKER_CASES[key] = Case(name, **dict(over))
    return _WORKER_CASES[key]


def _y_at_chunk(args):
    """Pool worker: the oracle outputs of one chunk of positions (each worker
    process builds the case once, from the workload name and overrides)."""
    name, over, pos = args
    return _worker_case(name, over).y_at(pos)


def _bwd_at_chunk(args):
    """Pool worker: the oracle's d hidden, de, dkv and scale terms at flat
    positions `pos`, given hidden rows at those positions and dy zero except at
    the ascending positions dy_pos (rows dy_val, storage form)."""
    name, over, pos, hid, dy_pos, dy_val = args
    c = _worker_case(name, over)
    T, D, K = c.T, c.w.conv_dilation, c.w.conv_kernel
    b, t = pos // T, pos % T
    ahead = np.unique(np.concatenate([(b * T + t + m * D)[t + m * D < T] for m in range(K)]))
    dy = np.zeros((len(ahead), c.w.hc_mult, c.w.hidden), dy_val.dtype)
    hit = np.isin(ahead, dy_pos)
    dy[hit] = dy_val[np.searchsorted(dy_pos, ahead[hit])]
    rows = c.rows_of(pos)
    gk, gq, cw = c.small
    return c.orc.backward_at(c.inp.ids, c.inp.remap, c.inp.table_rows(rows), c.wkv, gk, gq, cw, hid, dy, pos,
                             table_keys=rows, hidden_keys=pos, dy_keys=ahead, want_dkv=True, want_dgamma=True)


def _vg_at_chunk(args):
    """Pool worker: Vg = g V at flat positions `pos` -- the oracle's forward
    with every conv tap zero, which is Vg exactly (hidden rows given at the
    ascending positions `need` the conv would read)."""
    name, over, pos, need, hid = args
    c = _worker_case(name, over)
    rows = c.rows_of(need)
    gk, gq, cw = c.small
    return c.orc.forward_at(c.inp.ids, c.inp.remap, c.inp.table_rows(rows), c.wkv, gk, gq, np.zeros_like(cw), hid,
                            pos, table_keys=rows, hidden_keys=need)


def pool_map(fn, jobs):
    """map over a pool of spawned worker processes (serially with one worker)"""
    n = oracle_workers()
    if n == 1 or len(jobs) <= 1:
        return [fn(j) for j in jobs]
    ctx = multiprocessing.get_context("spawn")
    with concurrent.futures.ProcessPoolExecutor(min(n, len(jobs)), mp_context=ctx) as ex:
        return list(ex.map(fn, jobs))


class Case:
    def __init__(self, name: str, **over):
        self.name, self.over = name, tuple(sorted(over.items()))
        w = S.WORKLOADS[name]
        self.w = w.replace(**over) if over else w
        self.inp = S.Inputs(self.w)
        self.B = self.w.batch
        self.T = self.inp.seq_total            # whole sequence (prompt + steps for decode shapes)
        self.orc = orc.Oracle.from_workload(self.w, self.inp, batch=self.B, seqlen=self.T)
        self.off = np.concatenate([[0], np.cumsum(self.inp.primes)[:-1]]).astype(np.int64)

    # ---------------------------------------------------------------- host
    @functools.cached_property
    def idx(self) -> np.ndarray:
        """Oracle hash indices [B][T][H]."""
        return self.orc.hash(self.inp.ids, remap=self.inp.remap)

    @functools.cached_property
    def wkv(self):
        return self.inp.wkv()

    @functools.cached_property
    def small(self):
        return self.inp.gamma_k(), self.inp.gamma_q(), self.inp.conv_w()

    def rows_of(self, pos) -> np.ndarray:
        """Ascending stacked-table rows the positions' hashes select."""
        idx = self.idx.reshape(self.B * self.T, -1)[np.asarray(pos, dtype=np.int64)]
        return np.unique((idx + self.off).ravel())

    def e_at(self, pos) -> np.ndarray:
        """Oracle e rows (storage form) at flat positions."""
        idx = self.idx.reshape(self.B * self.T, -1)[pos]
        rows = np.unique((idx + self.off).ravel())
        return self.orc.with_shape(1, len(pos)).gather(self.inp.table_rows(rows), idx, keys=rows)

    def y_at(self, pos) -> np.ndarray:
        """Oracle outputs [len(pos)][hc][d] at flat positions b*T + t."""
        pos = np.asarray(pos, dtype=np.int64)
        need = orc.needed_positions(self.T, pos, self.w.conv_kernel, self.w.conv_dilation)
        idx = self.idx.reshape(self.B * self.T, -1)
        rows = np.unique((idx[need] + self.off).ravel())
        hid = self.inp.hidden_at(need // self.T, need % self.T).reshape(len(need), -1)
        gk, gq, cw = self.small
        return self.orc.forward_at(self.inp.ids, self.inp.remap, self.inp.table_rows(rows), self.wkv, gk, gq, cw,
                                   hid, pos, table_keys=rows, hidden_keys=need)

    def y_at_many(self, pos, chunk: int = 128) -> np.ndarray:
        """y_at over many positions, in contiguous chunks spread over a pool of
        fresh worker processes (spawned: they share nothing with this one)."""
        pos = np.asarray(pos, dtype=np.int64)
        n = oracle_workers()
        if n == 1 or len(pos) <= chunk:
            return self.y_at(pos)
        parts = np.array_split(pos, max(n, -(-len(pos) // chunk)))
        ctx = multiprocessing.get_context("spawn")
        with concurrent.futures.ProcessPoolExecutor(n, mp_context=ctx) as ex:
            out = list(ex.map(_y_at_chunk, [(self.name, self.over, p) for p in parts]))
        return np.concatenate(out)

    def sample_positions(self, n: int, seed: int = 0, head: int = 16) -> np.ndarray:
        """The first `head` positions of sequence 0, the last of the last sequence,
        and n seeded ones."""
        N = self.B * self.T
        rng = np.random.default_rng(seed)
        first = np.arange(min(head, self.T))
        last = np.array([N - 1])
        pick = rng.choice(N, size=min(n, N), replace=False)
        return np.unique(np.concatenate([first, last, pick]))

    # --------------------------------------------------------------- device
    @functools.cached_property
    def dev(self):
        from engram_synth.device import device_inputs

        return device_inputs(self.inp)

    def cfg(self, batch=None, seqlen=None):
        import hashed_gram_conditional_amd as eg

        return eg.EngramConfig.make(**self.w.config_kwargs(self.inp, batch=batch if batch is not None else self.B,
                                                            seqlen=seqlen if seqlen is not None else self.T))

    @functools.cached_property
    def params(self):
        import hashed_gram_conditional_amd as eg

        d = self.dev
        return eg.Params(remap=d["remap"], tables=d["tables"], w_kv=d["w_kv"], gamma_k=d["gamma_k"],
                         gamma_q=d["gamma_q"], conv_w=d["conv_w"])


def to_f64(t) -> np.ndarray:
    """Device tensor -> float64 numpy."""
    import torch

    return t.detach().to(torch.float64).cpu().numpy()


def sparse_dy_gradients(c: Case, hid: np.ndarray, P: np.ndarray, dy_val: np.ndarray, chunk: int = 16) -> dict:
    """The module's gradients over the whole batch for an upstream gradient dy
    that is zero except at the ascending flat positions P (rows dy_val, storage
    form), from the oracle at the positions whose gradients can be nonzero.

    Every step of the gradients is linear in dy, and position p's dKV reads dy
    only at p and D, 2D, ..., (K-1)D later in its sequence, so every per-token
    gradient vanishes outside P' = {p - jD}, and each sum over tokens is the sum
    over P':
      d_w_kv = sum_{p in P'} dkv[p] (x) e[p]; d_tables[row] = sum of de[p][head
      slice] over the p in P' hashing to row; d_gamma_k, d_gamma_q = the
      oracle's sums of the positions' terms; d_conv_w[h][c][j] = sum_{t in P}
      dy[t] Vg[t - (K-1-j)D], Vg from the oracle's forward with zero taps;
      d_hidden [N][hc][d], zero outside P'.
    hid: [N][hc][d] hidden states in storage form.  Returns float64 arrays
    keyed like engram_backward's outputs, plus "P'" (the positions) and "e"
    (their gathered rows as float64)."""
    import engram_synth as S

    w = c.w
    N, T, D, K, hc, d = c.B * c.T, c.T, w.conv_dilation, w.conv_kernel, w.hc_mult, w.hidden
    H, Dh = w.n_heads, w.head_dim
    P = np.asarray(P, dtype=np.int64)
    pb, pt = P // T, P % T
    Pext = np.unique(np.concatenate([(pb * T + pt - j * D)[pt - j * D >= 0] for j in range(K)]))
    hid = np.asarray(hid).reshape(N, hc, d)
    parts = np.array_split(Pext, max(1, -(-len(Pext) // chunk)))
    out = pool_map(_bwd_at_chunk, [(c.name, c.over, p, hid[p], P, dy_val) for p in parts])
    dkv = np.concatenate([o[2] for o in out]).reshape(len(Pext), -1)
    de = np.concatenate([o[1] for o in out])
    store = c.orc.store
    e = c.e_at(Pext)
    e64 = (e.astype(np.float32) if store == np.float32 else S.bf16_bits_to_f32(e)).astype(np.float64)
    ref = {"P'": Pext, "e": e64}
    ref["d_w_kv"] = dkv.T @ e64
    acc = np.zeros((w.table_rows, Dh))
    idx = c.idx.reshape(N, H)[Pext] + c.off[None, :]
    for h in range(H):
        np.add.at(acc, idx[:, h], de[:, h * Dh:(h + 1) * Dh])
    ref["d_tables"] = acc
    ref["d_gamma_k"] = sum(o[3] for o in out)
    ref["d_gamma_q"] = sum(o[4] for o in out)
    dh = np.zeros((N, hc, d))
    dh[Pext] = np.concatenate([o[0] for o in out])
    ref["d_hidden"] = dh
    # the taps: Vg at every position a tap of P reads
    taus = np.unique(np.concatenate([(pb * T + pt - (K - 1 - j) * D)[pt - (K - 1 - j) * D >= 0] for j in range(K)]))
    jobs = []
    for p in np.array_split(taus, max(1, -(-len(taus) // chunk))):
        tb, tt = p // T, p % T
        need = np.unique(np.concatenate([(tb * T + tt - m * D)[tt - m * D >= 0] for m in range(K)]))
        jobs.append((c.name, c.over, p, need, hid[need]))
    vg = np.concatenate(pool_map(_vg_at_chunk, jobs))
    dy64 = (dy_val.astype(np.float32) if store == np.float32 else S.bf16_bits_to_f32(dy_val)).astype(np.float64)
    dcw = np.zeros((hc, d, K))
    for j in range(K):
        tau_t = pt - (K - 1 - j) * D
        ok = tau_t >= 0
        dcw[:, :, j] = (dy64[ok] * vg[np.searchsorted(taus, pb[ok] * T + tau_t[ok])]).sum(axis=0)
    ref["d_conv_w"] = dcw
    return ref
