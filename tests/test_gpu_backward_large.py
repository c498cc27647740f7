"""engram_backward at B=8 T=4096 (bf16), the training step bench.py --train times.

The gradients of the tables' rows and of the hidden states belong to single
tokens (a token reads dy only at itself and D, 2D, 3D later), so the oracle
(orc_backward_at) evaluates them at chosen positions:
  - d hidden at 256 sampled positions;
  - table rows hit by 64 of those positions: each row's gradient is the sum
    of de over every token of the batch whose index is that row.
Gradients through the gate's score are compared where |s| >= 0.05 for the
tokens involved: the slope 1/(2 sqrt|s|) amplifies the rounding of s without
bound as s nears 0.  The weight, gamma and tap gradients are sums over the
whole batch; at this size they are checked by exact linearity in dy and by
the saved-activation path giving the same bits, and the weight gradient also
by an identity that ties it to the table rows' gradient."""
import concurrent.futures
import multiprocessing

import numpy as np
import pytest

from cases import TOL, Case, normwise, oracle_workers

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

NAME = "b8_t4096"
S_MIN = 0.05


@pytest.fixture(scope="module")
def eg():
    import hashed_gram_conditional_amd as m

    m.load()
    return m


@pytest.fixture(scope="module")
def case():
    return Case(NAME)


def _dy_dev(c):
    from engram_synth.device import fill

    dy = torch.empty_like(c.dev["hidden"])
    sid, sigma, bias = c.inp.recipe("dy")
    fill(dy, c.w.seed, sid, sigma, bias)
    return dy


_CASES: dict = {}


def _oracle_chunk(pos):
    """Pool worker: oracle d hidden, de and scores at flat positions (hidden and
    dy regenerated only at the rows those positions read)."""
    if NAME not in _CASES:
        _CASES[NAME] = Case(NAME)
    c = _CASES[NAME]
    pos = np.asarray(pos, dtype=np.int64)
    T, D, K = c.T, c.w.conv_dilation, c.w.conv_kernel
    b, t = pos // T, pos % T
    ahead = [b * T + t + m * D for m in range(K)]
    ahead = np.unique(np.concatenate([a[(a - b * T) < T] for a in ahead]))
    idx = c.idx.reshape(c.B * T, -1)
    rows = np.unique((idx[pos] + c.off).ravel())
    hid = c.inp.hidden_at(pos // T, pos % T)
    order = np.argsort(pos)
    hk, hid = pos[order], hid[order]
    dy = c.inp.dy_at(ahead // T, ahead % T)
    gk, gq, cw = c.small
    dh, de = c.orc.backward_at(c.inp.ids, c.inp.remap, c.inp.table_rows(rows), c.wkv, gk, gq, cw, hid, dy, pos,
                               table_keys=rows, hidden_keys=hk, dy_keys=ahead)
    kv = c.orc.project(c.wkv, c.orc.with_shape(1, len(pos)).gather(c.inp.table_rows(rows), idx[pos], keys=rows))
    _, s = c.orc.gate(gk, gq, kv, hid[np.argsort(order)], want_score=True)
    return dh, de, s


def _oracle(pos, chunk=32):
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
def run(eg, case):
    c = case
    dy = _dy_dev(c)
    dh, grads = eg.backward(c.cfg(), c.params, c.dev["ids"], c.dev["hidden"], dy)
    torch.cuda.synchronize()
    return dy, dh, grads


def test_d_hidden_at_sampled_positions(case, run):
    c = case
    _, dh, _ = run
    pos = c.sample_positions(240, seed=11)
    ref, _, s = _oracle(pos)
    got = dh.reshape(c.B * c.T, c.w.hc_mult, c.w.hidden)[torch.from_numpy(pos).cuda()].double().cpu().numpy()
    keep = np.abs(s) >= S_MIN
    assert keep.mean() > 0.8
    assert normwise(got[keep], ref[keep]) <= TOL["bf16"]


def test_table_rows_at_sampled_positions(case, run):
    """Rows of head h hit by sampled positions: the GPU's row gradient against
    the oracle's de of every token whose index is that row, summed."""
    c = case
    _, _, grads = run
    N, H, Dh = c.B * c.T, len(c.off), c.w.head_dim
    flat = (c.idx.reshape(N, H) + c.off[None, :])
    pos = np.random.default_rng(12).choice(N, 64, replace=False)
    rows = np.unique(flat[pos].ravel())
    hits = {int(r): [] for r in rows}
    for n, h in zip(*np.nonzero(np.isin(flat, rows))):
        hits[int(flat[n, h])].append((int(n), int(h)))
    # rows whose hitting tokens stay within a budget for the oracle
    keep = [r for r in rows if len(hits[int(r)]) <= 48]
    assert len(keep) >= len(rows) // 2
    toks = np.unique([n for r in keep for n, _ in hits[int(r)]])
    _, de, s = _oracle(toks)
    at = {int(n): i for i, n in enumerate(toks)}
    ok_tok = (np.abs(s) >= S_MIN).all(axis=1)
    sel, ref = [], []
    for r in keep:
        hs = hits[int(r)]
        if not all(ok_tok[at[n]] for n, _ in hs):
            continue
        sel.append(int(r))
        ref.append(sum(de[at[n], h * Dh:(h + 1) * Dh] for n, h in hs))
    assert len(sel) >= 100, (len(sel), len(keep))
    got = grads["d_tables"][torch.tensor(sel, device="cuda")].double().cpu().numpy()
    assert normwise(got, np.array(ref)) <= TOL["bf16"]
    # rows no token hits keep a zero gradient
    untouched = np.setdiff1d(np.arange(0, int(c.off[-1] + c.inp.primes[-1]), 997), flat.ravel())
    assert torch.count_nonzero(grads["d_tables"][torch.from_numpy(untouched).cuda()]).item() == 0


def test_gradients_are_linear_in_dy(eg, case, run):
    """2 dy is exact in bf16 and every step is linear in dy, so each gradient
    doubles bit for bit (the table rows within the rounding of the atomic
    adds' order)."""
    c = case
    dy, dh, grads = run
    dh2, g2 = eg.backward(c.cfg(), c.params, c.dev["ids"], c.dev["hidden"], dy * 2)
    torch.cuda.synchronize()
    assert torch.equal(dh2, dh * 2)
    for k in ("d_w_kv", "d_gamma_k", "d_gamma_q", "d_conv_w"):
        assert torch.equal(g2[k], grads[k] * 2), k
    t1, t2 = grads["d_tables"], g2["d_tables"]
    assert (t2 - 2 * t1).abs().max().item() <= 1e-5 * t1.abs().max().item()


def test_saved_activations_give_the_same_gradients(eg, case, run):
    c = case
    dy, dh, grads = run
    ws = eg.alloc_backward_workspace(c.cfg())
    eg.forward_train(c.cfg(), c.params, c.dev["ids"], c.dev["hidden"], ws)
    dh2, g2 = eg.backward_saved(c.cfg(), c.params, c.dev["hidden"], dy, ws)
    torch.cuda.synchronize()
    assert torch.equal(dh2, dh)
    for k in ("d_w_kv", "d_gamma_k", "d_gamma_q", "d_conv_w"):
        assert torch.equal(g2[k], grads[k]), k
    t1, t2 = grads["d_tables"], g2["d_tables"]
    assert (t2 - t1).abs().max().item() <= 1e-6 * t1.abs().max().item()


def _dot64(a, b, rows=1 << 20):
    """sum of a * b in float64, over row chunks (the tables are 3 GB in bf16)"""
    tot = torch.zeros((), dtype=torch.float64, device="cuda")
    for i in range(0, a.shape[0], rows):
        tot += (a[i:i + rows].double() * b[i:i + rows].double()).sum()
    return tot.item()


def test_weight_and_table_gradients_agree(eg, case):
    """<W_kv, dW_kv> = <tables, d_tables>: both are sum_t <dKV[t], W e[t]>.
    dW = sum_t dKV[t]^T e[t] comes from the weight GEMM over the token axis
    (here in split-K chunks), the table rows' gradient from de = dKV W
    scattered to the rows e came from: two independent paths.  With dy = y
    the sum is |y|^2 up to the epsilon of the key norm (y is linear in V, and
    the gates do not change when K is scaled), so it is large and positive and
    a wrong weight gradient cannot hide in cancellation."""
    c = case
    y = eg.forward(c.cfg(), c.params, c.dev["ids"], c.dev["hidden"])
    _, g = eg.backward(c.cfg(), c.params, c.dev["ids"], c.dev["hidden"], y)
    torch.cuda.synchronize()
    yy = _dot64(y.reshape(-1, c.w.hidden), y.reshape(-1, c.w.hidden))
    lhs = _dot64(c.dev["w_kv"], g["d_w_kv"])
    rhs = _dot64(c.dev["tables"], g["d_tables"])
    assert lhs > 0.5 * yy, (lhs, yy)
    assert abs(lhs - rhs) <= 1e-3 * abs(lhs), (lhs, rhs, yy)
