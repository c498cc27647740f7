"""The row-sparse table gradient (engram_backward_sparse, engram_backward_saved_sparse):
the rows a step's hashes select, once each and ascending, with their summed
gradients -- the training step of the B=1 T=32768 workload, whose 77 GB of
tables have no room for a dense float32 gradient.

  - small shapes: the rows equal the oracle's hashed rows (sorted, unique) bit
    for bit; their gradients equal the dense engram_backward's rows (the same
    de summed by atomics in another order) and the oracle's; every other
    gradient is bit-equal to the dense call's;
  - B=1 T=32768 after engram_forward_train: the rows bit for bit against the
    oracle's hash of every position; the gradients of rows hit by sampled
    positions against the oracle's de of every token hashing to them
    (orc_backward_at), and d hidden at sampled positions, where the gate's
    score is away from 0 (its slope 1/(2 sqrt|s|) amplifies the rounding of s).
"""
import concurrent.futures
import multiprocessing

import numpy as np
import pytest

from cases import TOL, Case, normwise, oracle_workers

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

S_MIN = 0.05


@pytest.fixture(scope="module")
def eg():
    import hashed_gram_conditional_amd as m

    m.load()
    return m


def _used_rows(c):
    return np.unique((c.idx.reshape(c.B * c.T, -1) + c.off[None, :]).ravel())


@pytest.mark.parametrize("name,over", [("tiny_fp32", {}), ("b4_t1024", dict(batch=2, seqlen=200, prime_base=4001))])
def test_sparse_rows_equal_dense_gradient(eg, name, over):
    c = Case(name, **over)
    cfg = c.cfg()
    hid = c.dev["hidden"]
    dy = torch.randn(hid.shape, generator=torch.Generator().manual_seed(9), dtype=torch.float32).to(hid.dtype).cuda()
    dh_d, g_d = eg.backward(cfg, c.params, c.dev["ids"], hid, dy)
    dh_s, g_s, rows = eg.backward_sparse(cfg, c.params, c.dev["ids"], hid, dy)
    torch.cuda.synchronize()
    n = int(rows["n_rows"].item())
    used = _used_rows(c)
    assert n == len(used)
    assert np.array_equal(rows["row_index"][:n].cpu().numpy(), used)
    dense_rows = g_d["d_tables"][rows["row_index"][:n]].double().cpu().numpy()
    got = rows["d_rows"][:n].double().cpu().numpy()
    assert np.abs(got - dense_rows).max() <= 1e-5 * np.abs(dense_rows).max()
    assert torch.equal(dh_s, dh_d)
    for k in ("d_w_kv", "d_gamma_k", "d_gamma_q", "d_conv_w"):
        assert torch.equal(g_s[k], g_d[k]), k
    # the dense gradient is zero off the used rows
    off = np.setdiff1d(np.arange(c.w.table_rows), used)
    assert torch.count_nonzero(g_d["d_tables"][torch.from_numpy(off).cuda()]).item() == 0


def test_sparse_saved_equals_recompute(eg):
    c = Case("b4_t1024", batch=2, seqlen=200, prime_base=4001)
    cfg = c.cfg()
    hid = c.dev["hidden"]
    dy = torch.randn(hid.shape, generator=torch.Generator().manual_seed(5), dtype=torch.float32).to(hid.dtype).cuda()
    ws = eg.alloc_backward_workspace(cfg)
    eg.forward_train(cfg, c.params, c.dev["ids"], hid, ws)
    d = c.dev
    no_tables = eg.Params(remap=d["remap"], tables=None, w_kv=d["w_kv"], gamma_k=d["gamma_k"], gamma_q=d["gamma_q"],
                          conv_w=d["conv_w"])
    dh_s, g_s, r_s = eg.backward_saved_sparse(cfg, no_tables, hid, dy, ws)
    dh_r, g_r, r_r = eg.backward_sparse(cfg, c.params, d["ids"], hid, dy)
    torch.cuda.synchronize()
    n = int(r_s["n_rows"].item())
    assert n == int(r_r["n_rows"].item())
    assert torch.equal(r_s["row_index"][:n], r_r["row_index"][:n])
    a, b = r_s["d_rows"][:n], r_r["d_rows"][:n]
    assert (a - b).abs().max().item() <= 1e-6 * b.abs().max().item()
    assert torch.equal(dh_s, dh_r)
    for k in ("d_w_kv", "d_gamma_k", "d_gamma_q", "d_conv_w"):
        assert torch.equal(g_s[k], g_r[k]), k


# ---------------------------------------------------------------- B=1 T=32768
NAME = "b1_t32768"
_CASES: dict = {}


def _large():
    if NAME not in _CASES:
        _CASES[NAME] = Case(NAME)
    return _CASES[NAME]


def _oracle_chunk(pos):
    """Pool worker: oracle d hidden, de and scores at flat positions (hidden and
    dy regenerated only at the rows those positions read)."""
    c = _large()
    pos = np.asarray(pos, dtype=np.int64)
    T, D, K = c.T, c.w.conv_dilation, c.w.conv_kernel
    b, t = pos // T, pos % T
    ahead = np.unique(np.concatenate([(b * T + t + m * D)[t + m * D < T] for m in range(K)]))
    idx = c.idx.reshape(c.B * T, -1)
    rows = np.unique((idx[pos] + c.off).ravel())
    order = np.argsort(pos)
    hid = c.inp.hidden_at(pos // T, pos % T)
    hk, hid_sorted = pos[order], hid[order]
    dy = c.inp.dy_at(ahead // T, ahead % T)
    gk, gq, cw = c.small
    dh, de = c.orc.backward_at(c.inp.ids, c.inp.remap, c.inp.table_rows(rows), c.wkv, gk, gq, cw, hid_sorted, dy,
                               pos, table_keys=rows, hidden_keys=hk, dy_keys=ahead)
    kv = c.orc.project(c.wkv, c.orc.with_shape(1, len(pos)).gather(c.inp.table_rows(rows), idx[pos], keys=rows))
    _, s = c.orc.gate(gk, gq, kv, hid, want_score=True)
    return dh, de, s


def _oracle(pos, chunk=8):
    pos = np.asarray(pos, dtype=np.int64)
    parts = np.array_split(pos, max(1, -(-len(pos) // chunk)))
    n = oracle_workers()
    if n == 1 or len(parts) == 1:
        out = [_oracle_chunk(p) for p in parts]
    else:
        with concurrent.futures.ProcessPoolExecutor(n, mp_context=multiprocessing.get_context("spawn")) as ex:
            out = list(ex.map(_oracle_chunk, parts))
    return tuple(np.concatenate([o[k] for o in out]) for k in range(3))


@pytest.fixture(scope="module")
def large_run(eg):
    from engram_synth.device import fill

    c = _large()
    cfg = c.cfg()
    dy = torch.empty_like(c.dev["hidden"])
    sid, sigma, bias = c.inp.recipe("dy")
    fill(dy, c.w.seed, sid, sigma, bias)
    ws = eg.alloc_backward_workspace(cfg)
    eg.forward_train(cfg, c.params, c.dev["ids"], c.dev["hidden"], ws)
    dh, grads, rows = eg.backward_saved_sparse(cfg, c.params, c.dev["hidden"], dy, ws)
    torch.cuda.synchronize()
    del ws, dy
    yield c, dh, grads, rows
    # release the device tables before the next module
    c.__dict__.pop("dev", None)
    c.__dict__.pop("params", None)
    torch.cuda.empty_cache()


def test_large_sparse_rows_are_the_hashed_rows(large_run):
    c, _, _, rows = large_run
    n = int(rows["n_rows"].item())
    used = _used_rows(c)
    assert n == len(used)
    assert np.array_equal(rows["row_index"][:n].cpu().numpy(), used)


def test_large_row_gradients_at_sampled_positions(large_run):
    """Rows hit by sampled positions (and by at most 48 tokens in all): the
    GPU's row gradient against the oracle's de of every token whose index is
    that row, summed."""
    c, _, _, rows = large_run
    N, H, Dh = c.B * c.T, len(c.off), c.w.head_dim
    flat = c.idx.reshape(N, H) + c.off[None, :]
    pos = np.random.default_rng(21).choice(N, 48, replace=False)
    cand = np.unique(flat[pos].ravel())
    hits = {int(r): [] for r in cand}
    for n_, h in zip(*np.nonzero(np.isin(flat, cand))):
        hits[int(flat[n_, h])].append((int(n_), int(h)))
    keep = [r for r in cand if len(hits[int(r)]) <= 48]
    assert len(keep) >= len(cand) // 2
    toks = np.unique([n_ for r in keep for n_, _ in hits[int(r)]])
    _, de, s = _oracle(toks)
    at = {int(n_): i for i, n_ in enumerate(toks)}
    ok_tok = (np.abs(s) >= S_MIN).all(axis=1)
    sel, ref = [], []
    for r in keep:
        hs = hits[int(r)]
        if not all(ok_tok[at[n_]] for n_, _ in hs):
            continue
        sel.append(int(r))
        ref.append(sum(de[at[n_], h * Dh:(h + 1) * Dh] for n_, h in hs))
    assert len(sel) >= 100, (len(sel), len(keep))
    n = int(rows["n_rows"].item())
    index = rows["row_index"][:n].cpu().numpy()
    slot = np.searchsorted(index, np.array(sel))
    assert np.array_equal(index[slot], np.array(sel))
    got = rows["d_rows"][torch.from_numpy(slot).cuda()].double().cpu().numpy()
    err = normwise(got, np.array(ref))
    assert err <= TOL["bf16"], err


def test_large_d_hidden_at_sampled_positions(large_run):
    c, dh, _, _ = large_run
    pos = c.sample_positions(96, seed=13)
    ref, _, s = _oracle(pos)
    got = dh.reshape(c.B * c.T, c.w.hc_mult, c.w.hidden)[torch.from_numpy(pos).cuda()].double().cpu().numpy()
    keep = np.abs(s) >= S_MIN
    assert keep.mean() > 0.8
    err = normwise(got[keep], ref[keep])
    assert err <= TOL["bf16"], err
