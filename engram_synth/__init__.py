"""Seeded synthetic inputs for the Engram forward pass.

This module holds no step of the method: it only draws random numbers and
shapes them into the inputs the method consumes (raw token ids, a compressed-id
remap table, hash multipliers, per-head prime moduli, embedding tables,
projection weights, RMSNorm scales, short-conv weights and hidden states).
Both the oracle side and the GPU side take their inputs from here.

Generator: the SplitMix64 output function ("mix64", Steele, Lea & Flood,
"Fast splittable pseudorandom number generators", OOPSLA 2014; public-domain
reference code by S. Vigna) used in counter mode.  Every array is a *stream*
with its own key; element i of a stream is

    key   = mix64(seed ^ (stream << 40))
    z_i   = mix64(key + (i + 1) * 0x9E3779B97F4A7C15)      (mod 2**64)

so any element can be regenerated on its own (the 77 GB table of the largest
workload is filled on the device by ``engram_synth.device`` with the same
definition, and the host regenerates only the rows it needs).

Real-valued arrays use an Irwin-Hall(4) draw of the four 16-bit lanes of z:
``v = f32(S - 131070) * f32(sigma * sqrt(3) / 65536) + f32(bias)`` in IEEE
float32 (one exact int->float conversion, one multiply, one add, no
contraction), then round-to-nearest-even to bfloat16 where the workload is
bf16.  Its mean is ``bias`` and its standard deviation ``sigma``; it stands in
for the normal draws the workloads name (a bounded near-normal, so that host
and device produce identical bits).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence

import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
IH4_CENTER = 131070          # mean of the sum of four uniform 16-bit lanes

# stream numbers (one per input array)
STREAM_TOKENS = 1        # Zipf uniforms for raw token ids
STREAM_RANK_PERM = 2     # rank -> raw id permutation (frequent ids are not small ids)
STREAM_REMAP_PERM = 3    # permutation that decides the surjective remap
STREAM_REMAP_TAIL = 4    # compressed id of each raw id beyond the first V'
STREAM_MULT = 5          # hash multipliers
STREAM_TABLE = 6         # multi-head embedding tables
STREAM_WKV = 7           # key projections (all branches) then value projection
STREAM_GAMMA_K = 8       # RMSNorm scale on keys
STREAM_GAMMA_Q = 9       # RMSNorm scale on queries
STREAM_CONV = 10         # short-conv taps
STREAM_HIDDEN = 11       # hidden states (queries)
STREAM_DY = 12           # upstream gradient of the module's output (backward tests)


def mix64(z: np.ndarray) -> np.ndarray:
    """SplitMix64 output function on a uint64 array (wrapping arithmetic)."""
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def stream_key(seed: int, stream: int) -> int:
    s = np.array([(seed ^ (stream << 40)) & 0xFFFFFFFFFFFFFFFF], dtype=np.uint64)
    return int(mix64(s)[0])


def stream_z(seed: int, stream: int, counters) -> np.ndarray:
    """z_i for the given element counters (int64/uint64 array-like)."""
    c = np.asarray(counters, dtype=np.uint64)
    key = np.uint64(stream_key(seed, stream))
    with np.errstate(over="ignore"):
        return mix64(key + (c + np.uint64(1)) * GOLDEN)


def ih4_scale(sigma: float) -> np.float32:
    return np.float32(sigma * math.sqrt(3.0) / 65536.0)


def ih4_values(seed: int, stream: int, counters, sigma: float, bias: float = 0.0) -> np.ndarray:
    """float32 Irwin-Hall(4) values of the given stream elements."""
    z = stream_z(seed, stream, counters)
    m = np.uint64(0xFFFF)
    s = ((z & m) + ((z >> np.uint64(16)) & m) + ((z >> np.uint64(32)) & m)
         + (z >> np.uint64(48))).astype(np.int64)
    v = (s - IH4_CENTER).astype(np.float32) * ih4_scale(sigma)
    return (v + np.float32(bias)).astype(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even float32 -> bfloat16, returned as uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def real_array(seed: int, stream: int, counters, sigma: float, bias: float, dtype: str) -> np.ndarray:
    """Stream elements in storage form: float32 array, or uint16 bf16 bits."""
    v = ih4_values(seed, stream, counters, sigma, bias)
    return v if dtype == "f32" else f32_to_bf16_bits(v)


# ---------------------------------------------------------------- integers
def primes_from(base: int, count: int) -> List[int]:
    """The `count` smallest primes >= base (trial division)."""
    out, n = [], max(2, base)
    while len(out) < count:
        if n < 4 or (n % 2 and all(n % q for q in range(3, int(math.isqrt(n)) + 1, 2))):
            out.append(n)
        n += 1
    return out


def zipf_cdf(vocab: int, a: float) -> np.ndarray:
    w = np.arange(1, vocab + 1, dtype=np.float64) ** (-a)
    c = np.cumsum(w)
    return c / c[-1]


def rank_permutation(seed: int, vocab: int) -> np.ndarray:
    z = stream_z(seed, STREAM_RANK_PERM, np.arange(vocab))
    return np.argsort(z, kind="stable").astype(np.int32)


def zipf_tokens(seed: int, vocab: int, a: float, shape: Sequence[int]) -> np.ndarray:
    """Raw token ids with a Zipf(a) rank law over [0, vocab), int32 of `shape`.

    Rank r (1-based) has probability proportional to r**-a; the rank is drawn by
    inverse CDF from the top 53 bits of z, and mapped to a raw id by a seeded
    permutation.
    """
    n = int(np.prod(shape)) if len(shape) else 1
    z = stream_z(seed, STREAM_TOKENS, np.arange(n))
    u = (z >> np.uint64(11)).astype(np.float64) * (1.0 / 9007199254740992.0)
    r = np.searchsorted(zipf_cdf(vocab, a), u, side="left")
    r = np.minimum(r, vocab - 1)
    return rank_permutation(seed, vocab)[r].reshape(shape).astype(np.int32)


def uniform_tokens(seed: int, vocab: int, shape: Sequence[int]) -> np.ndarray:
    n = int(np.prod(shape))
    z = stream_z(seed, STREAM_TOKENS, np.arange(n))
    return (z % np.uint64(vocab)).astype(np.int32).reshape(shape)


def make_remap(seed: int, vocab: int, vocab_c: int) -> np.ndarray:
    """Surjective raw -> compressed id table, int32 [vocab] with values in [0, vocab_c)."""
    perm = np.argsort(stream_z(seed, STREAM_REMAP_PERM, np.arange(vocab)), kind="stable")
    remap = np.empty(vocab, dtype=np.int32)
    remap[perm[:vocab_c]] = np.arange(vocab_c, dtype=np.int32)
    tail = np.arange(vocab_c, vocab)
    remap[perm[vocab_c:]] = (stream_z(seed, STREAM_REMAP_TAIL, tail) % np.uint64(vocab_c)).astype(np.int32)
    return remap


def make_multipliers(seed: int, max_order: int) -> np.ndarray:
    """Odd 64-bit multipliers m_k = 2 r + 1, r = z_k >> 2 (so m_k is in (0, 2**63))."""
    z = stream_z(seed, STREAM_MULT, np.arange(max_order))
    return ((z >> np.uint64(2)) * np.uint64(2) + np.uint64(1)).astype(np.int64)


# ---------------------------------------------------------------- workloads
@dataclasses.dataclass
class Workload:
    name: str
    batch: int
    seqlen: int
    vocab: int
    zipf_a: float
    orders: List[int]
    heads_per_order: int
    prime_base: int
    head_dim: int
    hidden: int
    hc_mult: int
    dtype: str                 # "f32" | "bf16"
    conv_kernel: int = 4
    conv_dilation: int = 0     # 0 -> max order
    pad_id: int = 0
    seed: int = 0
    decode_prompt: int = 0     # >0: decode-shaped workload
    decode_steps: int = 0
    sigma_table: float = 0.02
    sigma_w: float = 0.02
    sigma_gamma: float = 0.02
    sigma_conv: float = 0.02
    sigma_hidden: float = 1.0
    uniform_tokens: bool = False
    norm_eps: float = 1e-6
    gate_clamp: float = 1e-6

    def __post_init__(self):
        if self.conv_dilation == 0:
            self.conv_dilation = max(self.orders)

    @property
    def vocab_c(self) -> int:
        return (self.vocab * 77) // 100

    @property
    def max_order(self) -> int:
        return max(self.orders)

    @property
    def n_heads(self) -> int:
        return len(self.orders) * self.heads_per_order

    @property
    def emb_dim(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def primes(self) -> List[int]:
        return primes_from(self.prime_base, self.n_heads)

    @property
    def table_rows(self) -> int:
        return sum(self.primes)

    @property
    def tokens_per_call(self) -> int:
        return self.batch * self.seqlen

    def config_kwargs(self, inputs: "Inputs", batch: Optional[int] = None, seqlen: Optional[int] = None) -> dict:
        """Keyword arguments describing this workload's layer and call shape."""
        return dict(batch=self.batch if batch is None else batch, seqlen=self.seqlen if seqlen is None else seqlen,
                    vocab=self.vocab, orders=list(self.orders), heads_per_order=self.heads_per_order,
                    head_dim=self.head_dim, hidden=self.hidden, hc_mult=self.hc_mult,
                    multipliers=[int(m) for m in inputs.multipliers], primes=[int(p) for p in inputs.primes],
                    conv_kernel=self.conv_kernel, conv_dilation=self.conv_dilation, pad_id=self.pad_id,
                    dtype=self.dtype, norm_eps=self.norm_eps, gate_clamp=self.gate_clamp)

    def replace(self, **kw) -> "Workload":
        d = dataclasses.asdict(self)
        d.update(kw)
        if "orders" in kw and "conv_dilation" not in kw:
            d["conv_dilation"] = 0
        return Workload(**d)


WORKLOADS: Dict[str, Workload] = {
    "tiny_fp32": Workload("tiny_fp32", 1, 64, 1000, 1.1, [2, 3], 2, 1009, 16, 64, 1, "f32", seed=1001),
    "b4_t1024": Workload("b4_t1024", 4, 1024, 32000, 1.1, [2, 3], 8, 100003, 64, 1024, 4, "bf16", seed=1002),
    "b8_t4096": Workload("b8_t4096", 8, 4096, 129280, 1.1, [2, 3], 8, 1500000, 64, 2560, 4, "bf16", seed=1003),
    "decode_b256": Workload("decode_b256", 256, 1, 129280, 1.1, [2, 3], 8, 1500000, 64, 2560, 4, "bf16",
                            seed=1004, decode_prompt=16, decode_steps=512),
    "b1_t32768": Workload("b1_t32768", 1, 32768, 129280, 1.05, [2, 3, 4], 8, 20000000, 80, 4096, 4, "bf16",
                          seed=1005),
}


class Inputs:
    """Host-side generator of one workload's inputs.

    Small arrays are built eagerly; large ones (tables, weights, hidden) are
    produced on request, whole or at chosen element counters, so that a test
    can regenerate just the rows it needs.
    """

    def __init__(self, w: Workload):
        self.w = w
        s = w.seed
        self.remap = make_remap(s, w.vocab, w.vocab_c)
        self.multipliers = make_multipliers(s, w.max_order)
        self.primes = np.array(w.primes, dtype=np.int64)
        self.row_offset = np.concatenate([[0], np.cumsum(self.primes)[:-1]]).astype(np.int64)
        total = w.batch * (w.decode_prompt + w.decode_steps) if w.decode_prompt else w.batch * w.seqlen
        shape = (w.batch, w.decode_prompt + w.decode_steps) if w.decode_prompt else (w.batch, w.seqlen)
        if w.uniform_tokens:
            self.ids = uniform_tokens(s, w.vocab, shape)
        else:
            self.ids = zipf_tokens(s, w.vocab, w.zipf_a, shape)
        assert self.ids.size == total

    # element counts / shapes
    @property
    def seq_total(self) -> int:
        w = self.w
        return w.decode_prompt + w.decode_steps if w.decode_prompt else w.seqlen

    def table_shape(self):
        return (self.w.table_rows, self.w.head_dim)

    def wkv_shape(self):
        w = self.w
        return ((w.hc_mult + 1) * w.hidden, w.emb_dim)

    def hidden_shape(self):
        w = self.w
        return (w.batch, self.seq_total, w.hc_mult, w.hidden)

    # generators (storage form: float32, or uint16 bf16 bits)
    def table_rows(self, rows) -> np.ndarray:
        rows = np.asarray(rows, dtype=np.int64)
        dh = self.w.head_dim
        c = rows[:, None] * dh + np.arange(dh, dtype=np.int64)[None, :]
        return real_array(self.w.seed, STREAM_TABLE, c, self.w.sigma_table, 0.0, self.w.dtype)

    def table(self) -> np.ndarray:
        return self.table_rows(np.arange(self.w.table_rows))

    def wkv(self) -> np.ndarray:
        n = int(np.prod(self.wkv_shape()))
        return real_array(self.w.seed, STREAM_WKV, np.arange(n), self.w.sigma_w, 0.0,
                          self.w.dtype).reshape(self.wkv_shape())

    def gamma_k(self) -> np.ndarray:
        w = self.w
        return real_array(w.seed, STREAM_GAMMA_K, np.arange(w.hc_mult * w.hidden), w.sigma_gamma, 1.0,
                          w.dtype).reshape(w.hc_mult, w.hidden)

    def gamma_q(self) -> np.ndarray:
        w = self.w
        return real_array(w.seed, STREAM_GAMMA_Q, np.arange(w.hc_mult * w.hidden), w.sigma_gamma, 1.0,
                          w.dtype).reshape(w.hc_mult, w.hidden)

    def conv_w(self) -> np.ndarray:
        w = self.w
        n = w.hc_mult * w.hidden * w.conv_kernel
        return real_array(w.seed, STREAM_CONV, np.arange(n), w.sigma_conv, 0.0,
                          w.dtype).reshape(w.hc_mult, w.hidden, w.conv_kernel)

    def hidden_at(self, b, t) -> np.ndarray:
        """hidden[b, t] for index arrays b, t -> [len][hc][d] in storage form."""
        w = self.w
        b = np.asarray(b, dtype=np.int64)
        t = np.asarray(t, dtype=np.int64)
        per = w.hc_mult * w.hidden
        base = (b * self.seq_total + t) * per
        c = base[:, None] + np.arange(per, dtype=np.int64)[None, :]
        return real_array(w.seed, STREAM_HIDDEN, c, w.sigma_hidden, 0.0, w.dtype).reshape(
            len(b), w.hc_mult, w.hidden)

    def dy_at(self, b, t) -> np.ndarray:
        """An upstream gradient dL/dy at (b, t) for index arrays b, t -> [len][hc][d]
        in storage form (same shape and spread as the hidden states)."""
        w = self.w
        b = np.asarray(b, dtype=np.int64)
        t = np.asarray(t, dtype=np.int64)
        per = w.hc_mult * w.hidden
        base = (b * self.seq_total + t) * per
        c = base[:, None] + np.arange(per, dtype=np.int64)[None, :]
        return real_array(w.seed, STREAM_DY, c, w.sigma_hidden, 0.0, w.dtype).reshape(len(b), w.hc_mult, w.hidden)

    def hidden(self) -> np.ndarray:
        n = int(np.prod(self.hidden_shape()))
        return real_array(self.w.seed, STREAM_HIDDEN, np.arange(n), self.w.sigma_hidden, 0.0,
                          self.w.dtype).reshape(self.hidden_shape())

    # the (seed, stream, sigma, bias) recipe of each real array, for device fills
    def recipe(self, name: str):
        w = self.w
        return {
            "table": (STREAM_TABLE, w.sigma_table, 0.0),
            "wkv": (STREAM_WKV, w.sigma_w, 0.0),
            "gamma_k": (STREAM_GAMMA_K, w.sigma_gamma, 1.0),
            "gamma_q": (STREAM_GAMMA_Q, w.sigma_gamma, 1.0),
            "conv_w": (STREAM_CONV, w.sigma_conv, 0.0),
            "hidden": (STREAM_HIDDEN, w.sigma_hidden, 0.0),
            "dy": (STREAM_DY, w.sigma_hidden, 0.0),
        }[name]
