"""Pins of the oracle to the Engram pages and to mathematics (CPU only).

Each test fixes one step of the oracle to something other than the oracle
itself: a worked example or hand-derived value from the pages' definitions
(tests/golden/), a closed form, a library routine the step reduces to
(numpy int64 arithmetic, numpy matmul, torch rms_norm / conv1d / sigmoid),
brute force on tiny inputs, or an invariant the pages state (determinism,
causality).  The cases are chosen so that a dropped term, a wrong sign or
index, or a transposed operand in the oracle fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
MASK = (1 << 64) - 1


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def mk(B=1, T=8, orders=(2, 3), K=2, Dh=4, d=8, hc=1, mults=None, primes=None, pad=0, dtype="f32", ck=4, dil=None,
       eps=1e-6, clamp=1e-6, seed=0):
    rng = np.random.default_rng(seed)
    if mults is None:
        mults = [int(v) for v in rng.integers(-(2**63), 2**63 - 1, size=max(orders), dtype=np.int64)]
    if primes is None:
        primes = [101, 103, 107, 109, 113, 127, 131, 137, 139, 149, 151, 157][: len(orders) * K]
    return orc.Oracle(batch=B, seqlen=T, orders=list(orders), heads_per_order=K, head_dim=Dh, hidden=d, hc_mult=hc,
                      multipliers=mults, primes=primes, pad_id=pad, conv_kernel=ck, conv_dilation=dil, dtype=dtype,
                      norm_eps=eps, gate_clamp=clamp)


def brute_hash(x, orders, K, mults, primes, pad, hist=None):
    """Arbitrary-precision evaluation of the formula sheet's hash (sections 1.2-1.3, 4.2):
    the n-gram at t is [x[t], x[t-1], ..., x[t-n+1]] paired with m_0..m_{n-1}; products and
    xor taken mod 2**64, read as int64, then Python's floored %."""
    B, T = x.shape
    H = len(orders) * K
    out = np.zeros((B, T, H), np.int64)
    mo = max(orders)
    for b in range(B):
        for t in range(T):
            def tok(k):
                if t - k >= 0:
                    return int(x[b, t - k])
                if hist is not None:
                    return int(hist[b, mo - 1 + t - k])
                return pad
            h = 0
            for n in orders:
                mix = 0
                for k in range(n):
                    mix ^= (tok(k) * mults[k]) & MASK
                signed = mix - (1 << 64) if mix >= (1 << 63) else mix
                for j in range(K):
                    out[b, t, h] = signed % primes[h]
                    h += 1
    return out


# ------------------------------------------------------------------ shifts
def test_shift_worked_example(oracle_lib):
    g = load("shift_example.json")
    x = np.array([g["tokens"]], np.int32)
    o = mk(T=4, orders=(2, 3), pad=g["pad_id"])
    for k in range(3):
        assert o.shift(x, k).tolist() == [g[f"shift_{k}"]]
    i = g["trigram_position"]
    window = [int(o.shift(x, k)[0, i]) for k in (2, 1, 0)]
    assert window == g["trigram_window_oldest_first"]


def test_shift_reads_history_before_start(oracle_lib):
    o = mk(B=2, T=3, orders=(2, 4), pad=7)
    x = np.array([[1, 2, 3], [4, 5, 6]], np.int32)
    hist = np.array([[91, 92, 93], [94, 95, 96]], np.int32)       # oldest first, max_order-1 = 3
    assert o.shift(x, 3, hist).tolist() == [[91, 92, 93], [94, 95, 96]]
    assert o.shift(x, 1, hist).tolist() == [[93, 1, 2], [96, 4, 5]]
    assert o.shift(x, 2).tolist() == [[7, 7, 1], [7, 7, 4]]


# ------------------------------------------------------------------ hash
def test_hash_hand_vectors(oracle_lib):
    for v in load("hash_vectors.json")["vectors"]:
        mults = [int(m, 0) for m in v["multipliers"]]
        mults = [m - (1 << 64) if m >= (1 << 63) else m for m in mults]
        ids = np.array([v["ids"]], np.int32)
        o = mk(T=ids.shape[1], orders=v["orders"], K=len(v["primes"]) // len(v["orders"]), mults=mults,
               primes=v["primes"], pad=v["pad_id"])
        got = o.hash(ids)[0, v["position"]].tolist()
        assert got == v["idx"], v["name"]


@pytest.mark.parametrize("orders,K,pad,seed", [((2, 3), 2, 0, 1), ((1, 2, 4), 3, 5, 2), ((3,), 4, 0, 3),
                                               ((2, 3, 4, 5), 1, 11, 4)])
def test_hash_brute_force(oracle_lib, orders, K, pad, seed):
    rng = np.random.default_rng(seed)
    B, T = 3, 13
    primes = [int(p) for p in [1009, 1013, 1019, 1021, 2**31 - 1, 3, 2, 65537, 999983, 7, 11, 13, 17, 19, 23, 29]
              [: len(orders) * K]]
    o = mk(B=B, T=T, orders=orders, K=K, primes=primes, pad=pad, seed=seed)
    mults = list(o.cfg.multipliers)[: max(orders)]
    x = rng.integers(0, 2**31 - 1, size=(B, T)).astype(np.int32)
    x[0, :4] = [0, 1, 2, 3]
    assert np.array_equal(o.hash(x), brute_hash(x, orders, K, mults, primes, pad))
    hist = rng.integers(0, 1000, size=(B, max(orders) - 1)).astype(np.int32)
    assert np.array_equal(o.hash(x, hist=hist), brute_hash(x, orders, K, mults, primes, pad, hist))


def test_hash_matches_numpy_int64_semantics(oracle_lib):
    """The pages compute the mix with numpy int64 arrays; numpy's wrapping int64
    multiply, bitwise_xor and floored remainder are the library routine the hash
    reduces to."""
    rng = np.random.default_rng(7)
    B, T, orders, K = 2, 17, (2, 3), 3
    primes = [100003, 100019, 100043, 100049, 100057, 100069]
    o = mk(B=B, T=T, orders=orders, K=K, primes=primes, pad=0, seed=11)
    mults = np.array(list(o.cfg.multipliers)[:3], np.int64)
    x = rng.integers(0, 130000, size=(B, T)).astype(np.int64)
    shifted = [np.concatenate([np.zeros((B, k), np.int64), x[:, : T - k]], axis=1) for k in range(3)]
    expect = []
    with np.errstate(over="ignore"):
        for n in orders:
            prods = np.stack([shifted[k] * mults[k] for k in range(n)])
            mix = np.bitwise_xor.reduce(prods, axis=0)
            for j in range(K):
                expect.append(np.remainder(mix, primes[len(expect)]))
    expect = np.stack(expect, axis=-1)
    assert (expect >= 0).all()
    assert np.array_equal(o.hash(x.astype(np.int32)), expect)


def test_hash_range_determinism_and_batch_permutation(oracle_lib):
    rng = np.random.default_rng(3)
    o = mk(B=4, T=32, orders=(2, 3), K=4, seed=5)
    x = rng.integers(0, 50, size=(4, 32)).astype(np.int32)
    a = o.hash(x)
    assert np.array_equal(a, o.hash(x))
    p = np.array(list(o.cfg.primes)[:8])
    assert (a >= 0).all() and (a < p).all()
    perm = [2, 0, 3, 1]
    assert np.array_equal(o.hash(x[perm]), a[perm])


def test_hash_translation_invariance(oracle_lib):
    """The same n-gram always hashes to the same index (O(1) lookup property)."""
    o = mk(B=1, T=40, orders=(2, 3), K=2, seed=9)
    x = np.full((1, 40), 17, np.int32)
    w = [5, 9, 12]
    x[0, 10:13] = w
    x[0, 30:33] = w
    idx = o.hash(x)
    assert np.array_equal(idx[0, 12], idx[0, 32])          # both orders end at the same window
    assert np.array_equal(idx[0, 11, :2], idx[0, 31, :2])  # 2-gram (5, 9) at both places


def test_hash_dependency_structure(oracle_lib):
    """Order-n heads at t read exactly tokens t-n+1..t: a perturbation k back
    changes order-n heads only when k < n; a multiplier m_k only enters orders > k."""
    rng = np.random.default_rng(1)
    orders, K = (2, 3, 4), 2
    o = mk(B=1, T=20, orders=orders, K=K, seed=13)
    x = rng.integers(1, 1000, size=(1, 20)).astype(np.int32)
    base = o.hash(x)
    t = 12
    for k in range(5):
        y = x.copy()
        y[0, t - k] += 1
        d = o.hash(y)[0, t] != base[0, t]
        for oi, n in enumerate(orders):
            heads = d[oi * K:(oi + 1) * K]
            if k < n:
                assert heads.any(), (k, n)
            else:
                assert not heads.any(), (k, n)
    mults = list(o.cfg.multipliers)[:4]
    for k in range(4):
        m2 = mults.copy()
        m2[k] += 2
        o2 = mk(B=1, T=20, orders=orders, K=K, mults=m2, seed=13)
        d = (o2.hash(x)[0, t] != base[0, t])
        for oi, n in enumerate(orders):
            assert d[oi * K:(oi + 1) * K].any() == (k < n)


def test_hash_applies_remap(oracle_lib):
    rng = np.random.default_rng(2)
    o = mk(B=2, T=9, seed=3)
    remap = rng.integers(0, 40, size=100).astype(np.int32)
    ids = rng.integers(0, 100, size=(2, 9)).astype(np.int32)
    assert np.array_equal(o.hash(ids, remap=remap), o.hash(remap[ids]))
    with pytest.raises(orc.OracleError):
        o.hash(np.array([[100] * 9, [0] * 9], np.int32), remap=remap)


# ------------------------------------------------------------------ gather
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gather_rows_and_concatenation_order(oracle_lib, dtype):
    """Each table row encodes its own global row number, so any mistake in head
    offsets, row stride or concatenation order shows in the values."""
    orders, K, Dh = (2, 3), 3, 5
    primes = [11, 13, 17, 19, 23, 29]
    o = mk(B=2, T=6, orders=orders, K=K, Dh=Dh, primes=primes, dtype=dtype, seed=4)
    rows = sum(primes)
    val = (np.arange(rows)[:, None] * 8 + np.arange(Dh)[None, :]).astype(np.float32)
    table = val if dtype == "f32" else (val.view(np.uint32) >> 16).astype(np.uint16)
    if dtype == "bf16":
        val = (table.astype(np.uint32) << 16).view(np.float32)
    x = np.arange(12, dtype=np.int32).reshape(2, 6) * 7
    idx = o.hash(x)
    e = o.gather(table, idx.reshape(-1, 6))
    off = np.concatenate([[0], np.cumsum(primes)[:-1]])
    eb = e.view(np.float32) if dtype == "f32" else (e.astype(np.uint32) << 16).view(np.float32)
    eb = eb.reshape(12, 6, Dh)
    flat = idx.reshape(12, 6)
    for t in range(12):
        for h in range(6):
            assert np.array_equal(eb[t, h], val[off[h] + flat[t, h]])
    # sparse row source gives the same rows
    need = np.unique((flat + off[None, :]).ravel())
    e2 = o.gather(table[need], idx.reshape(-1, 6), keys=need)
    assert np.array_equal(e, e2)


# ------------------------------------------------------------------ projections
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_project_matches_numpy_matmul(oracle_lib, dtype):
    rng = np.random.default_rng(5)
    orders, K, Dh, d, hc = (2, 3), 2, 3, 5, 3        # E = 12 != d, hc + 1 = 4 blocks
    o = mk(orders=orders, K=K, Dh=Dh, d=d, hc=hc, dtype=dtype)
    E = 12
    w = rng.standard_normal(((hc + 1) * d, E)).astype(np.float32)
    e = rng.standard_normal((7, E)).astype(np.float32)
    if dtype == "bf16":
        wb = (w.view(np.uint32) >> 16).astype(np.uint16)
        eb = (e.view(np.uint32) >> 16).astype(np.uint16)
        w = (wb.astype(np.uint32) << 16).view(np.float32)
        e = (eb.astype(np.uint32) << 16).view(np.float32)
        kv = o.project(wb, eb)
    else:
        kv = o.project(w, e)
    ref = e.astype(np.float64) @ w.astype(np.float64).T
    np.testing.assert_allclose(kv.reshape(7, -1), ref, rtol=1e-12, atol=1e-12)
    # block layout: rows [h*d, (h+1)*d) of W give key h, the last block the value
    np.testing.assert_allclose(kv[:, hc], e.astype(np.float64) @ w[hc * d:].astype(np.float64).T, rtol=1e-12)


# ------------------------------------------------------------------ gate
def torch_gate(kv, hidden, gk, gq, d, hc, eps, clamp):
    """RMSNorm through torch's rms_norm, then the formula sheet's activation
    written with the torch ops it names (abs, clamp_min, sqrt, sign, sigmoid)."""
    K = torch.from_numpy(kv[:, :hc]).double()
    Q = torch.from_numpy(hidden).double()
    s = []
    for h in range(hc):
        kn = torch.nn.functional.rms_norm(K[:, h], (d,), torch.from_numpy(gk[h]).double(), eps)
        qn = torch.nn.functional.rms_norm(Q[:, h], (d,), torch.from_numpy(gq[h]).double(), eps)
        s.append((kn * qn).sum(-1) / math.sqrt(d))
    s = torch.stack(s, -1)
    g = (s.abs().clamp_min(clamp).sqrt() * s.sign()).sigmoid()
    return s.numpy(), g.numpy()


@pytest.mark.parametrize("eps", [1e-6, 0.3])
def test_gate_matches_torch_rms_norm(oracle_lib, eps):
    rng = np.random.default_rng(6)
    d, hc, n = 16, 3, 9
    o = mk(d=d, hc=hc, eps=eps)
    kv = rng.standard_normal((n, hc + 1, d)) * rng.uniform(0.01, 3, size=(n, hc + 1, 1))
    hid = rng.standard_normal((n, hc, d)).astype(np.float32)
    gk = rng.uniform(0.5, 1.5, size=(hc, d)).astype(np.float32)
    gq = rng.uniform(0.5, 1.5, size=(hc, d)).astype(np.float32)
    g, s = o.gate(gk, gq, kv, hid, want_score=True)
    s_ref, g_ref = torch_gate(kv, hid.astype(np.float64), gk.astype(np.float64), gq.astype(np.float64), d, hc, eps,
                              1e-6)
    np.testing.assert_allclose(s, s_ref, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(g, g_ref, rtol=1e-12, atol=1e-14)


def _gate1(o, K, Q, gk=None, gq=None):
    d = K.shape[-1]
    kv = np.zeros((1, 2, d))
    kv[0, 0] = K
    gk = np.ones((1, d), np.float32) if gk is None else gk
    gq = np.ones((1, d), np.float32) if gq is None else gq
    g, s = o.gate(gk, gq, kv, Q.reshape(1, 1, d).astype(np.float32), want_score=True)
    return float(s[0, 0]), float(g[0, 0])


def sig(a):
    return 1.0 / (1.0 + math.exp(-a))


def test_gate_closed_forms(oracle_lib):
    d = 64
    rng = np.random.default_rng(8)
    Q = rng.standard_normal(d).astype(np.float32)
    o = mk(d=d, eps=0.0)
    # K parallel to Q: normalised vectors coincide, s = sum(q^2/ms(q))/sqrt(d) = sqrt(d)
    s, g = _gate1(o, 3.0 * Q.astype(np.float64), Q)
    assert s == pytest.approx(math.sqrt(d), rel=1e-12)
    assert g == pytest.approx(sig(d ** 0.25), rel=1e-12)
    # anti-parallel: s = -sqrt(d), g = 1 - sigmoid(d^1/4)
    s, g = _gate1(o, -0.5 * Q.astype(np.float64), Q)
    assert s == pytest.approx(-math.sqrt(d), rel=1e-12)
    assert g == pytest.approx(1 - sig(d ** 0.25), rel=1e-12)
    # orthogonal: s = 0 and sign(0) = 0, so g = 1/2 exactly
    Kp = np.zeros(d)
    Kp[0], Kp[1] = Q[1], -Q[0]
    Qo = np.zeros(d, np.float32)
    Qo[0], Qo[1] = Q[0], Q[1]
    s, g = _gate1(o, Kp, Qo)
    assert s == 0.0 and g == 0.5
    # key scale drops out (RMSNorm), gamma_k = 2 doubles s
    s1, _ = _gate1(o, Q.astype(np.float64) + 0.1, Q)
    s2, _ = _gate1(o, 1000 * (Q.astype(np.float64) + 0.1), Q)
    assert s2 == pytest.approx(s1, rel=1e-12)
    s3, _ = _gate1(o, Q.astype(np.float64) + 0.1, Q, gk=np.full((1, d), 2.0, np.float32))
    assert s3 == pytest.approx(2 * s1, rel=1e-12)


def test_gate_epsilon_closed_form(oracle_lib):
    """Constant vectors K = c, Q = 1: s = sqrt(d) * c / sqrt((c^2 + eps) (1 + eps))."""
    d, eps = 16, 0.25
    o = mk(d=d, eps=eps)
    for c in (0.1, 1.0, -2.0):
        s, _ = _gate1(o, np.full(d, c), np.ones(d, np.float32))
        assert s == pytest.approx(math.sqrt(d) * c / math.sqrt((c * c + eps) * (1 + eps)), rel=1e-12)


def test_gate_activation_clamp_and_symmetry(oracle_lib):
    """g = sigmoid(sign(s) sqrt(max(|s|, 1e-6))): below the clamp g = sigmoid(+-1e-3);
    g(-s) = 1 - g(s); g is monotone in s."""
    d = 4
    o = mk(d=d, eps=0.0, clamp=1e-6)
    Q = np.array([1.0, 0.0, 0.0, 0.0], np.float32)
    vals = []
    for a in np.linspace(-1.0, 1.0, 41):
        # K = (a, sqrt(1-a^2), 0, 0), Q = e_0, eps = 0: both have rms 1/2, so s = (2a * 2) / sqrt(4) = 2a
        K = np.array([a, math.sqrt(max(0.0, 1 - a * a)), 0.0, 0.0])
        s, g = _gate1(o, K, Q)
        assert s == pytest.approx(2 * a, rel=1e-12, abs=1e-15)
        vals.append((s, g))
    vals.sort()
    gs = [g for _, g in vals]
    assert all(b >= a for a, b in zip(gs, gs[1:]))
    for s, g in vals:
        if s != 0.0:
            expect = sig(math.copysign(math.sqrt(max(abs(s), 1e-6)), s))
            assert g == pytest.approx(expect, rel=1e-12)
    # tiny positive and negative scores fall under the clamp
    K = np.array([1e-9, 1.0, 0.0, 0.0])
    s, g = _gate1(o, K, Q)
    assert 0 < s < 1e-6 and g == pytest.approx(sig(1e-3), rel=1e-12)
    s, g = _gate1(o, -K * np.array([1, -1, 1, 1]), Q)
    assert -1e-6 < s < 0 and g == pytest.approx(sig(-1e-3), rel=1e-12)


# ------------------------------------------------------------------ conv + residual
def test_conv_impulse_response(oracle_lib):
    """Vg = delta at t0: y[t0] = (1 + w3) delta, y[t0+jD] = w[3-j] delta, zero elsewhere."""
    B, T, d, hc, D = 1, 20, 3, 2, 3
    o = mk(B=B, T=T, d=d, hc=hc, dil=D)
    rng = np.random.default_rng(9)
    w = rng.standard_normal((hc, d, 4)).astype(np.float32)
    kv = np.zeros((B * T, hc + 1, d))
    t0 = 4
    kv[t0, hc, 1] = 1.0
    g = np.ones((B * T, hc))
    y = o.conv(w, kv, g)[0]
    expect = np.zeros((T, hc, d))
    expect[t0, :, 1] = 1.0 + w[:, 1, 3]
    for j in (1, 2, 3):
        expect[t0 + j * D, :, 1] = w[:, 1, 3 - j]
    np.testing.assert_allclose(y, expect, rtol=0, atol=1e-15)


def test_conv_zero_taps_is_identity_of_gated_value(oracle_lib):
    B, T, d, hc = 2, 7, 5, 3
    o = mk(B=B, T=T, d=d, hc=hc)
    rng = np.random.default_rng(10)
    kv = rng.standard_normal((B * T, hc + 1, d))
    g = rng.uniform(0, 1, size=(B * T, hc))
    y = o.conv(np.zeros((hc, d, 4), np.float32), kv, g)
    vg = g[:, :, None] * kv[:, hc][:, None, :]
    np.testing.assert_array_equal(y.reshape(B * T, hc, d), vg)


@pytest.mark.parametrize("K,D", [(4, 3), (4, 4), (3, 1), (1, 2)])
def test_conv_matches_torch_conv1d(oracle_lib, K, D):
    """Depthwise causal dilated conv = torch conv1d(groups = channels) with (K-1)*D
    zero padding on the left, cut to T, plus the residual."""
    B, T, d, hc = 2, 23, 6, 2
    o = mk(B=B, T=T, d=d, hc=hc, ck=K, dil=D)
    rng = np.random.default_rng(11)
    w = rng.standard_normal((hc, d, K)).astype(np.float32)
    kv = rng.standard_normal((B * T, hc + 1, d))
    g = rng.uniform(0, 1, size=(B * T, hc))
    y = o.conv(w, kv, g)
    vg = (g[:, :, None] * kv[:, hc][:, None, :]).reshape(B, T, hc * d)
    x = torch.from_numpy(vg).permute(0, 2, 1)                             # [B][C][T]
    wt = torch.from_numpy(w.astype(np.float64)).reshape(hc * d, 1, K)
    conv = torch.nn.functional.conv1d(x, wt, groups=hc * d, dilation=D, padding=(K - 1) * D)[..., :T]
    ref = (x + conv).permute(0, 2, 1).reshape(B, T, hc, d).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-13)


def test_conv_causality(oracle_lib):
    B, T, d, hc = 1, 30, 4, 2
    o = mk(B=B, T=T, d=d, hc=hc, dil=3)
    rng = np.random.default_rng(12)
    w = rng.standard_normal((hc, d, 4)).astype(np.float32)
    kv = rng.standard_normal((T, hc + 1, d))
    g = rng.uniform(0, 1, size=(T, hc))
    y = o.conv(w, kv, g)
    i = 17
    kv2, g2 = kv.copy(), g.copy()
    kv2[i + 1:] += 1.0
    g2[i + 1:] *= 0.5
    y2 = o.conv(w, kv2, g2)
    np.testing.assert_array_equal(y[0, : i + 1], y2[0, : i + 1])
    assert not np.allclose(y[0, i + 1], y2[0, i + 1])


# ------------------------------------------------------------------ whole forward
def small_case(B=2, T=21, orders=(2, 3), K=2, Dh=4, d=8, hc=2, dtype="f32", seed=21, V=60, Vc=37, pad=0):
    rng = np.random.default_rng(seed)
    o = mk(B=B, T=T, orders=orders, K=K, Dh=Dh, d=d, hc=hc, dtype=dtype, pad=pad, seed=seed,
           primes=[31, 37, 41, 43, 47, 53, 59, 61][: len(orders) * K])
    E = len(orders) * K * Dh
    rows = sum(list(o.cfg.primes)[: len(orders) * K])

    def real(*shape, scale=1.0, loc=0.0):
        a = (loc + scale * rng.standard_normal(shape)).astype(np.float32)
        return a if dtype == "f32" else (a.view(np.uint32) >> 16).astype(np.uint16)

    args = dict(ids=rng.integers(0, V, size=(B, T)).astype(np.int32),
                remap=rng.integers(0, Vc, size=V).astype(np.int32),
                table=real(rows, Dh, scale=0.5), w_kv=real((hc + 1) * d, E, scale=0.3),
                gamma_k=real(hc, d, scale=0.1, loc=1.0), gamma_q=real(hc, d, scale=0.1, loc=1.0),
                conv_w=real(hc, d, 4, scale=0.5), hidden=real(B, T, hc, d))
    return o, args


def as64(a, dtype):
    return a.astype(np.float64) if dtype == "f32" else (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_forward_matches_library_composition(oracle_lib, dtype):
    """Whole forward against an independent float64 composition: brute-force hash,
    numpy fancy-index gather, numpy matmul, torch rms_norm gate, torch conv1d."""
    B, T, orders, K, Dh, d, hc = 2, 21, (2, 3), 2, 4, 8, 2
    o, a = small_case(B, T, orders, K, Dh, d, hc, dtype)
    y = o.forward(**a)
    primes = list(o.cfg.primes)[:4]
    x = a["remap"][a["ids"]]
    idx = brute_hash(x, orders, K, list(o.cfg.multipliers)[:3], primes, 0)
    off = np.concatenate([[0], np.cumsum(primes)[:-1]])
    tab = as64(a["table"], dtype)
    e = tab[(idx + off).reshape(-1)].reshape(B * T, -1)
    kv = (e @ as64(a["w_kv"], dtype).T).reshape(B * T, hc + 1, d)
    _, g = torch_gate(kv, as64(a["hidden"], dtype).reshape(B * T, hc, d), as64(a["gamma_k"], dtype),
                      as64(a["gamma_q"], dtype), d, hc, 1e-6, 1e-6)
    vg = (g[:, :, None] * kv[:, hc][:, None, :]).reshape(B, T, hc * d)
    xt = torch.from_numpy(vg).permute(0, 2, 1)
    wt = torch.from_numpy(as64(a["conv_w"], dtype)).reshape(hc * d, 1, 4)
    ref = (xt + torch.nn.functional.conv1d(xt, wt, groups=hc * d, dilation=3, padding=9)[..., :T])
    ref = ref.permute(0, 2, 1).reshape(B, T, hc, d).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-11, atol=1e-12)


def test_forward_causality_and_batch_independence(oracle_lib):
    o, a = small_case(B=2, T=25)
    y = o.forward(**a)
    i = 14
    b = dict(a)
    b["ids"] = a["ids"].copy()
    b["ids"][:, i + 1:] = (b["ids"][:, i + 1:] + 1) % 60
    b["hidden"] = a["hidden"].copy()
    b["hidden"][:, i + 1:] *= 2
    y2 = o.forward(**b)
    np.testing.assert_array_equal(y[:, : i + 1], y2[:, : i + 1])
    assert not np.allclose(y[:, i + 1:], y2[:, i + 1:])
    # each sequence alone gives the same rows
    o1 = o.with_shape(1, 25)
    for s in range(2):
        one = {k: (v[s:s + 1] if k in ("ids", "hidden") else v) for k, v in a.items()}
        np.testing.assert_array_equal(o1.forward(**one)[0], y[s])


def test_forward_at_matches_full_forward(oracle_lib):
    o, a = small_case(B=3, T=30, dtype="bf16", seed=4)
    y = o.forward(**a)
    pos = np.array([0, 1, 2, 9, 10, 29, 30, 31, 45, 89])
    ya = o.forward_at(a["ids"], a["remap"], a["table"], a["w_kv"], a["gamma_k"], a["gamma_q"], a["conv_w"],
                      a["hidden"], pos)
    np.testing.assert_array_equal(ya, y.reshape(-1, *y.shape[2:])[pos])
    # the same from sparse row sources that hold only what those outputs read
    need = orc.needed_positions(30, pos, 4, 3)
    idx = o.hash(a["ids"], remap=a["remap"]).reshape(90, -1)
    off = np.concatenate([[0], np.cumsum(list(o.cfg.primes)[:4])[:-1]])
    rows = np.unique((idx[need] + off).ravel())
    hid = a["hidden"].reshape(90, -1)
    yb = o.forward_at(a["ids"], a["remap"], a["table"][rows], a["w_kv"], a["gamma_k"], a["gamma_q"], a["conv_w"],
                      hid[need], pos, table_keys=rows, hidden_keys=need)
    np.testing.assert_array_equal(yb, ya)


def test_forward_rejects_bad_config(oracle_lib):
    with pytest.raises(ValueError):
        mk(orders=(2, 3), mults=[1, 3])
    o = mk(orders=(3, 2))
    with pytest.raises(orc.OracleError):
        o.hash(np.zeros((1, 8), np.int32))


def test_oracle_pool_matches_serial():
    """The process-pool evaluation used by the large parity tests returns the
    serial oracle's values, bit for bit, in position order."""
    from cases import Case

    c = Case("tiny_fp32")
    pos = np.arange(c.B * c.T)[::-1].copy()
    assert np.array_equal(c.y_at_many(pos, chunk=8), c.y_at(pos))
