"""GPU parity: every C-ABI call against the oracle on the seeded workloads.

Bars: hash indices and gathered rows bit-exact; outputs within max|y - y_ref| /
max|y_ref| <= 1e-5 on the float32 workload and <= 2e-2 on the bf16 ones.
"""
import numpy as np
import pytest

from cases import TOL, Case, normwise, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def eg():
    import hashed_gram_conditional_amd as m

    m.load()
    return m


_cases = {}


def case(name, **over):
    key = (name, repr(sorted(over.items())))
    if key not in _cases:
        _cases[key] = Case(name, **over)
    return _cases[key]


def sync():
    torch.cuda.synchronize()


# ------------------------------------------------------------------ inputs
@pytest.mark.parametrize("name", ["tiny_fp32", "b4_t1024"])
def test_device_fill_matches_host_generator(eg, name):
    from engram_synth.device import storage_numpy

    c = case(name)
    d = c.dev
    rng = np.random.default_rng(0)
    rows = rng.choice(c.w.table_rows, size=64, replace=False)
    assert np.array_equal(storage_numpy(d["tables"])[rows], c.inp.table_rows(rows))
    assert np.array_equal(storage_numpy(d["w_kv"]), c.wkv)
    gk, gq, cw = c.small
    assert np.array_equal(storage_numpy(d["gamma_k"]), gk)
    assert np.array_equal(storage_numpy(d["conv_w"]), cw)
    hb = rng.integers(0, c.B, 8)
    ht = rng.integers(0, c.T, 8)
    assert np.array_equal(storage_numpy(d["hidden"])[hb, ht], c.inp.hidden_at(hb, ht))


# ------------------------------------------------------------------ hash
@pytest.mark.parametrize("name", ["tiny_fp32", "b4_t1024", "b8_t4096"])
def test_hash_bit_exact(eg, name):
    c = case(name)
    idx = eg.engram_hash(c.cfg(), c.params, c.dev["ids"])
    sync()
    assert np.array_equal(idx.cpu().numpy().astype(np.int64), c.idx)


def test_hash_edge_cases(eg):
    c = case("tiny_fp32")
    p = c.params
    ids = c.dev["ids"]
    # ragged lengths, T shorter than the largest order, a single token
    for T in (1, 2, 3, 17, 63):
        got = eg.engram_hash(c.cfg(1, T), p, ids[:, :T].contiguous())
        sync()
        assert np.array_equal(got.cpu().numpy(), c.orc.with_shape(1, T).hash(c.inp.ids[:, :T], remap=c.inp.remap))
    # empty calls enqueue nothing and succeed
    eg.engram_hash(c.cfg(0, 64), p, ids)
    eg.engram_hash(c.cfg(1, 0), p, ids)
    # out-of-range raw ids hash as pad_id
    bad = c.inp.ids.copy()
    bad[0, [5, 40]] = [-3, c.w.vocab + 7]
    got = eg.engram_hash(c.cfg(), p, torch.from_numpy(bad).cuda())
    sync()
    x = c.inp.remap[np.clip(bad, 0, c.w.vocab - 1)]
    x[0, [5, 40]] = c.w.pad_id
    assert np.array_equal(got.cpu().numpy(), c.orc.hash(x))


def test_hash_negative_multipliers_and_pad(eg):
    """Multipliers across the whole int64 range (negative mixes) and a nonzero pad."""
    import hashed_gram_conditional_amd as m
    import oracle as orc

    rng = np.random.default_rng(5)
    mults = [int(v) for v in rng.integers(-(2**63), 2**63 - 1, size=4, dtype=np.int64)]
    primes = [2, 3, 1009, 65537, 2147483647, 999983]
    kw = dict(batch=3, seqlen=45, orders=[1, 2, 4], heads_per_order=2, head_dim=8, hidden=8, hc_mult=1,
              multipliers=mults, primes=primes, pad_id=123456)
    cfg = m.EngramConfig.make(vocab=1 << 30, dtype="f32", **kw)
    o = orc.Oracle(dtype="f32", **kw)
    ids = rng.integers(0, 1 << 30, size=(3, 45)).astype(np.int32)
    tables = torch.zeros((8, 8), device="cuda")
    p = m.Params(tables=tables, w_kv=tables, gamma_k=tables, gamma_q=tables, conv_w=tables)
    got = m.engram_hash(cfg, p, torch.from_numpy(ids).cuda())
    sync()
    assert np.array_equal(got.cpu().numpy(), o.hash(ids))


def test_hash_with_a_compressed_vocabulary(eg):
    """The remap built from token texts (compressed ids: NFKC, lower case,
    accents removed, equal keys merged) drives the hash: bit-exact against the
    oracle's hash with the oracle's own compressed ids."""
    import oracle as orc
    from engram_synth.vocab import synthetic_vocab
    from hashed_gram_conditional_amd.compressed_vocab import build_remap
    from oracle.compressed_vocab import compressed_ids

    c = case("b4_t1024")
    texts = synthetic_vocab(c.w.seed, c.w.vocab)
    remap, n = build_remap(texts)
    ref_remap, n_ref = compressed_ids(texts)
    assert n == n_ref
    d = c.dev
    p = eg.Params(remap=torch.from_numpy(remap).cuda(), tables=d["tables"], w_kv=d["w_kv"], gamma_k=d["gamma_k"],
                  gamma_q=d["gamma_q"], conv_w=d["conv_w"])
    got = eg.engram_hash(c.cfg(), p, d["ids"])
    sync()
    o = orc.Oracle.from_workload(c.w, c.inp, batch=c.B, seqlen=c.T)
    assert np.array_equal(got.cpu().numpy().astype(np.int64),
                          o.hash(c.inp.ids, remap=np.asarray(ref_remap, dtype=np.int32)))


# ------------------------------------------------------------------ gather
@pytest.mark.parametrize("name", ["tiny_fp32", "b4_t1024", "b8_t4096"])
def test_gather_bit_exact(eg, name):
    from engram_synth.device import storage_numpy

    c = case(name)
    idx = eg.engram_hash(c.cfg(), c.params, c.dev["ids"])
    e = eg.engram_gather(c.cfg(), c.params, idx)
    sync()
    N = c.B * c.T
    pos = np.arange(N)           # every position
    got = storage_numpy(e).reshape(N, -1)[pos]
    assert np.array_equal(got, c.e_at(pos))


# ------------------------------------------------------------------ projections
@pytest.mark.parametrize("name", ["tiny_fp32", "b4_t1024"])
def test_project_within_tolerance(eg, name):
    c = case(name)
    idx = eg.engram_hash(c.cfg(), c.params, c.dev["ids"])
    e = eg.engram_gather(c.cfg(), c.params, idx)
    kv = eg.engram_project(c.cfg(), c.params, e)
    sync()
    from engram_synth.device import storage_numpy

    N = c.B * c.T
    pos = np.arange(N) if N <= 64 else c.sample_positions(128, seed=2)
    e_np = storage_numpy(e).reshape(N, -1)[pos]
    ref = c.orc.project(c.wkv, e_np)
    err = normwise(to_f64(kv).reshape(N, -1)[pos], ref.reshape(len(pos), -1))
    # bf16: one rounding of a float32-accumulated dot product (relative 2^-9) bounds it
    assert err <= (1e-6 if c.w.dtype == "f32" else 4e-3), err


@pytest.mark.parametrize("shape", [(3, 77, 2, 3, 8, 40, 2), (1, 300, 3, 1, 16, 24, 3), (2, 129, 2, 4, 16, 136, 1)])
def test_project_ragged_tiles(eg, shape):
    """Token, channel and reduction counts that are not multiples of the GEMM tiles."""
    import hashed_gram_conditional_amd as m
    import oracle as orc

    B, T, n_orders, K, Dh, d, hc = shape
    orders = list(range(2, 2 + n_orders))
    H = n_orders * K
    E = H * Dh
    rng = np.random.default_rng(sum(shape))
    kw = dict(batch=B, seqlen=T, orders=orders, heads_per_order=K, head_dim=Dh, hidden=d, hc_mult=hc,
              multipliers=[3, 5, 7, 9, 11], primes=[101 + 2 * i for i in range(H)])
    for dtype in ("f32", "bf16"):
        cfg = m.EngramConfig.make(vocab=1000, dtype=dtype, **kw)
        o = orc.Oracle(dtype=dtype, **kw)
        w = rng.standard_normal(((hc + 1) * d, E)).astype(np.float32)
        e = rng.standard_normal((B * T, E)).astype(np.float32)
        if dtype == "bf16":
            wt = torch.from_numpy(w).to(torch.bfloat16)
            et = torch.from_numpy(e).to(torch.bfloat16)
        else:
            wt, et = torch.from_numpy(w), torch.from_numpy(e)
        from engram_synth.device import storage_numpy

        ref = o.project(storage_numpy(wt), storage_numpy(et)).reshape(B * T, -1)
        wt, et = wt.cuda(), et.cuda()
        p = m.Params(tables=wt, w_kv=wt, gamma_k=wt, gamma_q=wt, conv_w=wt)
        kv = m.engram_project(cfg, p, et)
        sync()
        err = normwise(to_f64(kv).reshape(B * T, -1), ref)
        assert err <= (1e-6 if dtype == "f32" else 4e-3), (dtype, err)


# ------------------------------------------------------------------ gate + conv
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("strong", [False, True])
def test_gate_conv_with_oracle_kv(eg, dtype, strong):
    """Gate, conv and residual alone, fed the oracle's projections; strong conv
    taps and spread gammas make a dropped or shifted tap show."""
    import hashed_gram_conditional_amd as m
    import oracle as orc
    from engram_synth.device import storage_numpy

    B, T, d, hc, D = 2, 70, 48, 3, 3
    rng = np.random.default_rng(7 + strong)
    kw = dict(batch=B, seqlen=T, orders=[2, 3], heads_per_order=1, head_dim=8, hidden=d, hc_mult=hc,
              multipliers=[3, 5, 7], primes=[11, 13])
    cfg = m.EngramConfig.make(vocab=10, dtype=dtype, **kw)
    o = orc.Oracle(dtype=dtype, **kw)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    kv = torch.from_numpy(rng.standard_normal((B, T, hc + 1, d)).astype(np.float32) * 0.02).to(tdt)
    hid = torch.from_numpy(rng.standard_normal((B, T, hc, d)).astype(np.float32)).to(tdt)
    sc = 0.5 if strong else 0.02
    cw = torch.from_numpy(rng.standard_normal((hc, d, 4)).astype(np.float32) * sc).to(tdt)
    lo, hi = (0.5, 1.5) if strong else (0.98, 1.02)
    gk = torch.from_numpy(rng.uniform(lo, hi, (hc, d)).astype(np.float32)).to(tdt)
    gq = torch.from_numpy(rng.uniform(lo, hi, (hc, d)).astype(np.float32)).to(tdt)
    kv_ref = (kv.to(torch.float64).numpy()).reshape(B * T, hc + 1, d)
    g_ref = o.gate(storage_numpy(gk), storage_numpy(gq), kv_ref, storage_numpy(hid).reshape(B * T, hc, d))
    y_ref = o.conv(storage_numpy(cw), kv_ref, g_ref)
    dv = {k: v.cuda() for k, v in dict(kv=kv, hid=hid, cw=cw, gk=gk, gq=gq).items()}
    p = m.Params(tables=dv["kv"], w_kv=dv["kv"], gamma_k=dv["gk"], gamma_q=dv["gq"], conv_w=dv["cw"])
    y, g = m.engram_gate_conv(cfg, p, dv["kv"], dv["hid"])
    sync()
    assert normwise(to_f64(g).reshape(B * T, hc), g_ref) <= 1e-5
    assert normwise(to_f64(y), y_ref) <= TOL[dtype] / (4 if dtype == "bf16" else 1)


# ------------------------------------------------------------------ whole forward
@pytest.mark.parametrize("name,n", [("tiny_fp32", None), ("b4_t1024", None), ("b8_t4096", 1024)])
def test_forward_within_tolerance(eg, name, n):
    """Every position of the small workloads; at B=8, T=4096 the first 16
    positions (the pad and zero-history edge), the last one and 1024 seeded."""
    c = case(name)
    y = eg.forward(c.cfg(), c.params, c.dev["ids"], c.dev["hidden"])
    sync()
    N = c.B * c.T
    pos = np.arange(N) if n is None else c.sample_positions(n, seed=3)
    ref = c.y_at_many(pos)
    err = normwise(to_f64(y).reshape(N, c.w.hc_mult, c.w.hidden)[pos], ref)
    assert err <= TOL[c.w.dtype], err


# every count at its maximum: 8 orders (1..8) of 8 heads = 64 heads, 16 branches, 8 taps
MAXIMAL = dict(orders=[1, 2, 3, 4, 5, 6, 7, 8], heads_per_order=8, head_dim=8, hidden=128, hc_mult=16,
               conv_kernel=8, conv_dilation=8, prime_base=4001)


@pytest.mark.parametrize("over,fused", [
    (dict(batch=2, seqlen=100, hidden=200, hc_mult=3), False),   # d % 128 != 0: stored projections + gate kernel
    (dict(batch=3, seqlen=77, hidden=256, hc_mult=2), True),     # fused GEMM with a ragged token count
    (dict(batch=1, seqlen=300, hidden=384, hc_mult=1, orders=[2, 3, 4], conv_dilation=4), True),
    (dict(batch=2, seqlen=2000), True),   # key channels 256-wide, then the value channels as a plain GEMM
    (dict(batch=1, seqlen=130, hidden=96, hc_mult=8), False),    # 8 branches; 24 of a wavefront's 64 lanes in the conv
    (dict(batch=2, seqlen=61, hidden=256, hc_mult=6, conv_kernel=3, conv_dilation=2), True),   # 6 branches
    (dict(batch=2, seqlen=90, hidden=128, hc_mult=2, conv_kernel=1), True),    # one tap: no history
    (dict(batch=1, seqlen=150, hidden=256, conv_kernel=8, conv_dilation=5), True),   # the largest conv
    (dict(MAXIMAL, batch=2, seqlen=40), True),   # 8 orders x 8 heads, 16 branches, 8 taps at dilation 8
    (dict(batch=5, seqlen=1), True),   # one token per sequence, no state: only the current tap
    (dict(batch=3, seqlen=2), True),   # sequences shorter than the dilation (3)
])
def test_forward_paths_on_ragged_shapes(eg, over, fused):
    c = case("b4_t1024", **over)
    names = eg.kernel_names(c.cfg())
    assert (names[1] == "project_gate_gemm") == fused, names
    assert ("project_value_gemm" in names) == (c.B * c.T == 4000), names
    y = eg.forward(c.cfg(), c.params, c.dev["ids"], c.dev["hidden"])
    sync()
    N = c.B * c.T
    pos = np.arange(N)
    err = normwise(to_f64(y).reshape(N, c.w.hc_mult, c.w.hidden)[pos], c.y_at_many(pos))
    assert err <= TOL["bf16"], err


def test_forward_is_deterministic(eg):
    c = case("b4_t1024")
    ws = eg.alloc_workspace(c.cfg())
    y1 = eg.forward(c.cfg(), c.params, c.dev["ids"], c.dev["hidden"], workspace=ws).clone()
    y2 = eg.forward(c.cfg(), c.params, c.dev["ids"], c.dev["hidden"], workspace=ws)
    sync()
    assert torch.equal(y1, y2)


def test_forward_errors(eg):
    import hashed_gram_conditional_amd as m

    c = case("tiny_fp32")
    cfg = c.cfg()
    ws = eg.alloc_workspace(cfg)
    with pytest.raises(m.EngramError) as ei:
        eg.forward(cfg, c.params, c.dev["ids"], c.dev["hidden"], workspace=ws[:128])
    assert ei.value.status == -2
    bad = c.cfg()
    bad.orders[1] = 2            # not ascending
    with pytest.raises(m.EngramError) as ei:
        eg.forward(bad, c.params, c.dev["ids"], c.dev["hidden"], workspace=ws)
    assert ei.value.status == -1
    # empty batch succeeds without work
    eg.forward(c.cfg(0, 64), c.params, c.dev["ids"], c.dev["hidden"], workspace=ws)


# ------------------------------------------------------------------ state: chunked prefill and decode
def test_chunked_prefill_matches_single_prefill(eg):
    c = case("b4_t1024")
    full = eg.forward(c.cfg(), c.params, c.dev["ids"], c.dev["hidden"])
    st = eg.State(c.cfg(), c.B)
    outs = []
    t0 = 0
    for L in (1, 2, 7, 100, 300, 614):
        ids = c.dev["ids"][:, t0:t0 + L].contiguous()
        hid = c.dev["hidden"][:, t0:t0 + L].contiguous()
        outs.append(eg.forward(c.cfg(c.B, L), c.params, ids, hid, state=st))
        t0 += L
    sync()
    assert t0 == c.T
    chunked = torch.cat(outs, dim=1)
    assert torch.equal(chunked, full)
    assert st.n_past.cpu().tolist() == [c.T] * c.B


def test_chunks_with_the_largest_conv_match_single_prefill(eg):
    """8 taps at dilation 5: the state's rings hold 36 positions, and chunks
    shorter than the history (1, 3) read most of it from the rings."""
    c = case("b4_t1024", batch=3, seqlen=140, hidden=256, conv_kernel=8, conv_dilation=5)
    full = eg.forward(c.cfg(), c.params, c.dev["ids"], c.dev["hidden"])
    st = eg.State(c.cfg(), c.B)
    outs, t0 = [], 0
    for L in (1, 3, 40, 1, 95):
        ids = c.dev["ids"][:, t0:t0 + L].contiguous()
        hid = c.dev["hidden"][:, t0:t0 + L].contiguous()
        outs.append(eg.forward(c.cfg(c.B, L), c.params, ids, hid, state=st))
        t0 += L
    sync()
    assert t0 == c.T
    assert torch.equal(torch.cat(outs, dim=1), full)


def test_chunks_with_every_count_at_its_maximum_match_single_prefill(eg):
    """64 heads of orders up to 8 (a 7-token history from the token ring), 16
    branches, 8 taps at dilation 8 (57-slot rings), in chunks of 1 to 30 tokens."""
    c = case("b4_t1024", **dict(MAXIMAL, batch=2, seqlen=64))
    full = eg.forward(c.cfg(), c.params, c.dev["ids"], c.dev["hidden"])
    st = eg.State(c.cfg(), c.B)
    outs, t0 = [], 0
    for L in (1, 2, 5, 1, 25, 30):
        ids = c.dev["ids"][:, t0:t0 + L].contiguous()
        hid = c.dev["hidden"][:, t0:t0 + L].contiguous()
        outs.append(eg.forward(c.cfg(c.B, L), c.params, ids, hid, state=st))
        t0 += L
    sync()
    assert t0 == c.T
    assert torch.equal(torch.cat(outs, dim=1), full)
    pos = np.arange(c.B * c.T)
    err = normwise(to_f64(full).reshape(c.B * c.T, c.w.hc_mult, c.w.hidden), c.y_at_many(pos))
    assert err <= TOL["bf16"], err


@pytest.mark.parametrize("hc,hidden", [(1, 128), (3, 256), (16, 128)])
def test_decode_steps_with_any_branch_count_match_single_prefill(eg, hc, hidden):
    """Single-token steps run decode_tail, whose workgroups hold one wavefront
    per branch (64 to 1024 threads): 1, 3 and 16 branches, bit-equal to one
    prefill over the same tokens."""
    c = case("b4_t1024", batch=3, seqlen=24, hidden=hidden, hc_mult=hc)
    assert eg.kernel_names(c.cfg(c.B, 1), with_state=True)[-1] == "decode_tail"
    full = eg.forward(c.cfg(), c.params, c.dev["ids"], c.dev["hidden"])
    st = eg.State(c.cfg(), c.B)
    outs, t0 = [], 0
    for L in (5, 1, 1, 1, 3, 1, 1, 1, 1, 1, 1, 7):
        ids = c.dev["ids"][:, t0:t0 + L].contiguous()
        hid = c.dev["hidden"][:, t0:t0 + L].contiguous()
        outs.append(eg.forward(c.cfg(c.B, L), c.params, ids, hid, state=st))
        t0 += L
    sync()
    assert t0 == c.T
    assert torch.equal(torch.cat(outs, dim=1), full)


def test_long_chunks_match_single_prefill(eg):
    """Chunks of more than 16384 tokens each take the conv's long walks, whose
    history at the chunk start comes from the state's rings; T = 2100 leaves a
    ragged last run (walks cover 16 x 3 positions)."""
    c = case("b4_t1024", batch=16, seqlen=2100)
    full = eg.forward(c.cfg(), c.params, c.dev["ids"], c.dev["hidden"])
    st = eg.State(c.cfg(), c.B)
    outs, t0 = [], 0
    for L in (1040, 1060):
        assert c.B * L >= 16384
        ids = c.dev["ids"][:, t0:t0 + L].contiguous()
        hid = c.dev["hidden"][:, t0:t0 + L].contiguous()
        outs.append(eg.forward(c.cfg(c.B, L), c.params, ids, hid, state=st))
        t0 += L
    sync()
    assert torch.equal(torch.cat(outs, dim=1), full)
    pos = c.sample_positions(256, seed=11)
    err = normwise(to_f64(full).reshape(c.B * c.T, c.w.hc_mult, c.w.hidden)[pos], c.y_at_many(pos))
    assert err <= TOL["bf16"], err


def test_decode_matches_oracle(eg):
    """Decode-shaped workload: prompt prefill, then 512 single-token steps with
    state; for 8 seeded sequences every position's output must equal the
    oracle's prefill over the whole sequence."""
    c = case("decode_b256")
    w = c.w
    P = w.decode_prompt
    cfgp = c.cfg(c.B, P)
    cfg1 = c.cfg(c.B, 1)
    ids, hid = c.dev["ids"], c.dev["hidden"]
    st = eg.State(cfg1, c.B)
    ws = eg.alloc_workspace(cfgp)
    outs = [eg.forward(cfgp, c.params, ids[:, :P].contiguous(), hid[:, :P].contiguous(), state=st, workspace=ws)]
    steps_ids = ids[:, P:].t().contiguous()
    steps_hid = hid[:, P:].transpose(0, 1).contiguous()
    for s in range(w.decode_steps):
        outs.append(eg.forward(cfg1, c.params, steps_ids[s], steps_hid[s], state=st, workspace=ws))
    sync()
    y = torch.cat(outs, dim=1)                                   # [B][P+steps][hc][d]
    # equals one prefill over the whole sequence on the GPU, up to bf16 output
    # rounding: a step of 256 tokens and the whole prefill may pick different
    # GEMM channel tiles, which sum the gate's partial sums in another order
    whole = eg.forward(c.cfg(), c.params, ids, hid)
    sync()
    assert normwise(to_f64(y), to_f64(whole)) <= 1e-2
    rng = np.random.default_rng(4)
    b = np.sort(rng.choice(c.B, size=8, replace=False))
    pos = (b[:, None] * c.T + np.arange(c.T)[None, :]).ravel()
    ref = c.y_at_many(pos)
    got = to_f64(y).reshape(c.B * c.T, w.hc_mult, w.hidden)[pos]
    assert normwise(got, ref) <= TOL[w.dtype]


def _hash_with_history(c, ids_chunk, t0):
    """The oracle's hash of a chunk that starts at position t0 of every
    sequence, given as history the compressed ids of the max_order - 1
    positions before it (pad before the sequence start)."""
    W = c.w.max_order - 1
    x = c.inp.remap[c.inp.ids]
    hist = np.full((c.B, W), c.w.pad_id, dtype=np.int32)
    for k in range(1, W + 1):
        if t0 - k >= 0:
            hist[:, W - k] = x[:, t0 - k]
    L = ids_chunk.shape[1]
    return c.orc.with_shape(c.B, L).hash(ids_chunk, remap=c.inp.remap, hist=hist)


def test_decode_state_hash_and_gather_bit_exact(eg):
    """Decode-shaped workload, the state path of the hash: the prompt's prefill
    and each of the 512 single-token steps hash with the state (the tokens
    before the step come from the state's token ring) and gather their rows
    before the forward advances the state.  Every sequence's indices over all
    528 positions equal the oracle's hash of the whole sequence, each step's
    equal the oracle's hash of that step alone given the ids before it as
    history, and the gathered rows equal the oracle's gather, bit for bit."""
    from engram_synth.device import storage_numpy

    c = case("decode_b256")
    w = c.w
    P, steps = w.decode_prompt, w.decode_steps
    cfgp, cfg1 = c.cfg(c.B, P), c.cfg(c.B, 1)
    ids, hid = c.dev["ids"], c.dev["hidden"]
    st = eg.State(cfg1, c.B)
    ws = eg.alloc_workspace(cfgp)
    idx = [eg.engram_hash(cfgp, c.params, ids[:, :P].contiguous(), state=st)]
    e = [eg.engram_gather(cfgp, c.params, idx[0])]
    eg.forward(cfgp, c.params, ids[:, :P].contiguous(), hid[:, :P].contiguous(), state=st, workspace=ws)
    steps_ids = ids[:, P:].t().contiguous()
    steps_hid = hid[:, P:].transpose(0, 1).contiguous()
    for s in range(steps):
        i1 = eg.engram_hash(cfg1, c.params, steps_ids[s], state=st)
        idx.append(i1)
        e.append(eg.engram_gather(cfg1, c.params, i1))
        eg.forward(cfg1, c.params, steps_ids[s], steps_hid[s], state=st, workspace=ws)
    sync()
    got = torch.cat([i.reshape(c.B, -1, c.w.n_heads) for i in idx], dim=1).cpu().numpy().astype(np.int64)
    assert got.shape == c.idx.shape
    assert np.array_equal(got, c.idx)
    for s in (0, 1, 2, 3, 100, steps - 1):
        t0 = P + s
        ref = _hash_with_history(c, c.inp.ids[:, t0:t0 + 1], t0)
        assert np.array_equal(idx[1 + s].cpu().numpy().reshape(c.B, 1, -1).astype(np.int64), ref), s
    rows = np.concatenate([storage_numpy(x).reshape(c.B, -1, c.w.emb_dim) for x in e], axis=1)
    rows = rows.reshape(c.B * c.T, -1)
    for b0 in range(0, c.B, 64):     # every position, 64 sequences at a time
        pos = np.arange(b0 * c.T, (b0 + 64) * c.T)
        assert np.array_equal(rows[pos], c.e_at(pos)), b0


def test_chunked_hash_and_gather_bit_exact(eg):
    """Chunked prefill, the state path of the hash for chunks longer than one
    token: each chunk's indices, hashed with the state before the forward
    advances it, equal the oracle's hash of the chunk given the ids before it
    as history, and its rows the oracle's gather; with orders up to 8 (a
    7-token history from the ring) as well."""
    from engram_synth.device import storage_numpy

    for name, over, lens in (("b4_t1024", {}, (1, 2, 7, 100, 300, 614)),
                             ("b4_t1024", dict(MAXIMAL, batch=2, seqlen=64), (1, 2, 5, 1, 25, 30))):
        c = case(name, **over)
        st = eg.State(c.cfg(), c.B)
        t0 = 0
        for L in lens:
            ids = c.dev["ids"][:, t0:t0 + L].contiguous()
            hid = c.dev["hidden"][:, t0:t0 + L].contiguous()
            cfg = c.cfg(c.B, L)
            idx = eg.engram_hash(cfg, c.params, ids, state=st)
            e = eg.engram_gather(cfg, c.params, idx)
            eg.forward(cfg, c.params, ids, hid, state=st)
            sync()
            got = idx.cpu().numpy().astype(np.int64)
            assert np.array_equal(got, _hash_with_history(c, c.inp.ids[:, t0:t0 + L], t0)), (name, t0, L)
            assert np.array_equal(got, c.idx[:, t0:t0 + L]), (name, t0, L)
            pos = (np.arange(c.B)[:, None] * c.T + np.arange(t0, t0 + L)[None, :]).ravel()
            assert np.array_equal(storage_numpy(e).reshape(c.B * L, -1), c.e_at(pos)), (name, t0, L)
            t0 += L
        assert t0 == c.T


def test_decode_state_copy_resumes(eg):
    """Checkpoint and resume of the decode state: after k steps the state is
    copied; the remaining steps run from the original and from the copy give
    identical outputs and end at the same position."""
    c = case("decode_b256")
    P, k, n = c.w.decode_prompt, 5, 12
    cfgp, cfg1 = c.cfg(c.B, P), c.cfg(c.B, 1)
    ids, hid = c.dev["ids"], c.dev["hidden"]
    steps_ids = ids[:, P:].t().contiguous()
    steps_hid = hid[:, P:].transpose(0, 1).contiguous()
    ws = eg.alloc_workspace(cfgp)
    st = eg.State(cfg1, c.B)
    eg.forward(cfgp, c.params, ids[:, :P].contiguous(), hid[:, :P].contiguous(), state=st, workspace=ws)
    for s in range(k):
        eg.forward(cfg1, c.params, steps_ids[s], steps_hid[s], state=st, workspace=ws)
    copy = st.clone()
    a = [eg.forward(cfg1, c.params, steps_ids[s], steps_hid[s], state=st, workspace=ws).clone() for s in range(k, n)]
    b = [eg.forward(cfg1, c.params, steps_ids[s], steps_hid[s], state=copy, workspace=ws).clone() for s in range(k, n)]
    sync()
    assert all(torch.equal(x, y) for x, y in zip(a, b))
    assert torch.equal(st.n_past, copy.n_past)
    assert st.n_past.cpu().tolist() == [P + n] * c.B


# ------------------------------------------------------------------ several layers
def test_hash_layers_equal_single_layer_hashes(eg):
    """One pass over three layers (each with its own multipliers) gives, for
    every layer, the oracle's indices with that layer's multipliers; also
    continuing a state."""
    import dataclasses

    import engram_synth as S
    import oracle as orc

    c = case("b4_t1024")
    rng = np.random.default_rng(11)
    mults = [S.make_multipliers(1002 + 7919 * l, c.w.max_order).tolist() for l in range(3)]
    mults[2][0] = -(2**63) + 12345      # full int64 range, negative
    got = eg.engram_hash_layers(c.cfg(), c.params, c.dev["ids"], mults)
    sync()
    for l in range(3):
        o = orc.Oracle.from_workload(c.w, c.inp, batch=c.B, seqlen=c.T)
        o.cfg.multipliers[:len(mults[l])] = mults[l]
        ref = o.hash(c.inp.ids, remap=c.inp.remap)
        assert np.array_equal(got[l].cpu().numpy(), ref), l
    # continuing a state after a 100-token prefill
    st = eg.State(c.cfg(), c.B)
    eg.forward(c.cfg(c.B, 100), c.params, c.dev["ids"][:, :100].contiguous(), c.dev["hidden"][:, :100].contiguous(),
               state=st)
    ids2 = c.dev["ids"][:, 100:140].contiguous()
    got2 = eg.engram_hash_layers(c.cfg(c.B, 40), c.params, ids2, mults, state=st)
    for l in range(3):
        cfg = c.cfg(c.B, 40)
        for k in range(len(mults[l])):
            cfg.multipliers[k] = ctypes_i64(mults[l][k])
        one = eg.engram_hash(cfg, c.params, ids2, state=st)
        sync()
        assert torch.equal(got2[l], one), l


def ctypes_i64(v):
    import ctypes

    return ctypes.c_int64(int(v)).value


# ------------------------------------------------------------------ kernel counts, debug build
@pytest.mark.parametrize("name,over,T", [("b4_t1024", dict(batch=2, seqlen=100, hidden=200, hc_mult=3), None),
                                         ("decode_b256", {}, 16), ("decode_b256", {}, 1), ("b4_t1024", {}, None)])
def test_timed_forward_counts_the_kernels_it_names(eg, name, over, T):
    """engram_forward_timed reports as many kernels as engram_forward_kernel_name
    names, on every plan: stored projections, the fused projection, the decode
    tail, and the split projection; with and without a state."""
    c = case(name, **over)
    T = c.T if T is None else T
    cfg = c.cfg(c.B, T)
    ids = c.dev["ids"][:, :T].contiguous()
    hid = c.dev["hidden"][:, :T].contiguous()
    plans = set()
    for with_state in (False, True):
        st = eg.State(cfg, c.B) if with_state else None
        names = eg.kernel_names(cfg, with_state=with_state)
        _, nk = eg.forward_timed(cfg, c.params, ids, hid, [], state=st)
        sync()
        assert nk == len(names), (names, nk)
        plans.add(tuple(names))
    assert len(plans) == 2


def test_debug_build_rejects_out_of_range_ids(eg):
    """The ENGRAM_DEBUG build checks the raw ids on the host: an id outside
    [0, vocab) makes engram_hash and engram_forward return ENGRAM_EINVAL with
    nothing enqueued (the release build hashes it as pad_id); valid ids give the
    release build's indices."""
    import ctypes

    import hashed_gram_conditional_amd as m

    dbg = m.load(debug=True)
    c = case("tiny_fp32")
    cfg = c.cfg()
    out = torch.full((c.B, c.T, c.w.n_heads), -1, dtype=torch.int32, device="cuda")
    args = lambda ids: (ctypes.byref(cfg), ctypes.byref(c.params._c), ctypes.c_void_p(ids.data_ptr()), None,
                        ctypes.c_void_p(out.data_ptr()), None)
    assert dbg.engram_hash(*args(c.dev["ids"])) == 0
    sync()
    assert torch.equal(out, eg.engram_hash(cfg, c.params, c.dev["ids"]))
    for v in (-1, c.w.vocab):
        bad = c.dev["ids"].clone()
        bad[0, 7] = v
        out.fill_(-1)
        assert dbg.engram_hash(*args(bad)) == -1
        sync()
        assert bool((out == -1).all())
        ws = eg.alloc_workspace(cfg)
        y = torch.empty((c.B, c.T, c.w.hc_mult, c.w.hidden), dtype=torch.float32, device="cuda")
        rc = dbg.engram_forward(ctypes.byref(cfg), ctypes.byref(c.params._c), ctypes.c_void_p(bad.data_ptr()),
                                ctypes.c_void_p(c.dev["hidden"].data_ptr()), None, ctypes.c_void_p(y.data_ptr()),
                                ctypes.c_void_p(ws.data_ptr()), ws.numel(), None)
        assert rc == -1
