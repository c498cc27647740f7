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


def _y_at_chunk(args):
    """Pool worker: the oracle outputs of one chunk of positions (each worker
    process builds the case once, from the workload name and overrides)."""
    name, over, pos = args
    key = (name, repr(over))
    if key not in _WORKER_CASES:
        _WORKER_CASES[key] = Case(name, **dict(over))
    return _WORKER_CASES[key].y_at(pos)


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
