"""engram_backward's sums over the token axis against the oracle, at a shape
whose weight gradient takes the split-K path.

dW = sum_t dKV[t] (x) e[t] over N tokens is computed in S independent chunks of
the token axis whose products are then added in chunk order; the gammas' and
taps' gradients are per-block partial sums added in block order.  The split
only pays once the product has few output tiles and a long token axis, so the
smallest shape that takes it still sums over 32768 tokens: here hc = 4 branches
of d = 512 (2560 output rows) by 32 heads of 64 (E = 2048) over 16 sequences of
2048 tokens, which the library splits in 8 chunks of 4096 tokens.

The upstream gradient dy is zero except at 128 positions P (the first and last
token of every chunk, every sequence start and end, and seeded ones).  Each
step of the gradients is linear in dy, and a token's dKV reads dy only at itself
and D, 2D, ..., (K-1)D later, so every per-token gradient vanishes outside
P' = {p - jD}: the oracle evaluates the gradients at P' alone (orc_backward_at),
and the sums over the whole batch are the sums over P':
  - d_w_kv  = sum_{p in P'} dkv[p] (x) e[p]           (dkv from the oracle, e its gather)
  - d_tables[row] = sum of de[p][head slice] over the p in P' hashing to row
  - d_gamma_k, d_gamma_q: the oracle's sums of the positions' terms
  - d_conv_w[h][c][j] = sum_{t in P} dy[t] Vg[t - (K-1-j)D], Vg from the
    oracle's forward with zero taps (which is Vg exactly)
  - d_hidden at P', and exactly zero elsewhere.
The GPU still runs every kernel over all 32768 tokens; the zero terms add
exact zeros to its sums.  At P' the hidden states are each branch's +-
normalised key plus noise, so the gate's score is far from zero where the
gradient passes through it (its slope 1/(2 sqrt|s|) is unbounded at 0).
"""
import numpy as np
import pytest

from cases import TOL, Case, normwise, sparse_dy_gradients

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

NAME = "b4_t1024"
OVER = dict(batch=16, seqlen=2048, hidden=512, hc_mult=4, heads_per_order=16, prime_base=4001)
CHUNK = 4096     # tokens per split-K chunk at this shape


@pytest.fixture(scope="module")
def eg():
    import hashed_gram_conditional_amd as m

    m.load()
    return m


def k_splits(M, N, K):
    """The split count the library's weight-gradient product takes for an M x N
    output over K tokens (the cost model of its split-K planner: rounds of
    256 x 256 tiles over 256 compute units, times the depth per split)."""
    tiles = -(-M // 256) * -(-N // 256)
    best, best_cost = 1, float(-(-tiles // 256))
    for S in range(2, 9):
        if K // S < 4096 or S * tiles < 512:
            continue
        cost = -(-S * tiles // 256) / S
        if cost < 0.9 * best_cost:
            best, best_cost = S, cost
    return best


@pytest.fixture(scope="module")
def setup(eg):
    import engram_synth as S
    from engram_synth.device import storage_numpy

    c = Case(NAME, **OVER)
    w = c.w
    N, T, D, K, hc, d = c.B * c.T, c.T, w.conv_dilation, w.conv_kernel, w.hc_mult, w.hidden
    assert k_splits((hc + 1) * d, w.emb_dim, N) == N // CHUNK == 8
    rng = np.random.default_rng(17)
    # P: both ends of every chunk and of every sequence, and seeded positions
    edges = np.unique(np.concatenate([np.arange(0, N, CHUNK), np.arange(CHUNK - 1, N, CHUNK), np.arange(0, N, T),
                                      np.arange(T - 1, N, T)]))
    P = np.unique(np.concatenate([edges, rng.choice(np.setdiff1d(np.arange(N), edges), 128 - len(edges),
                                                    replace=False)]))
    pb, pt = P // T, P % T
    Pext = np.unique(np.concatenate([(pb * T + pt - j * D)[pt - j * D >= 0] for j in range(K)]))
    # hidden: the synthetic states, except at P' +- each branch's normalised key plus noise
    hid = storage_numpy(c.dev["hidden"]).reshape(N, hc, d).copy()
    e64 = S.bf16_bits_to_f32(c.e_at(Pext)).astype(np.float64)
    Kx = (e64 @ S.bf16_bits_to_f32(c.wkv[: hc * d]).astype(np.float64).T).reshape(len(Pext), hc, d)
    sign = np.where(rng.random((len(Pext), hc, 1)) < 0.5, -1.0, 1.0)
    aligned = sign * Kx / np.sqrt((Kx ** 2).mean(-1, keepdims=True)) + 0.3 * rng.standard_normal(Kx.shape)
    hid[Pext] = S.f32_to_bf16_bits(aligned.astype(np.float32))
    dy_val = S.f32_to_bf16_bits(rng.standard_normal((len(P), hc, d)).astype(np.float32))
    dy = np.zeros((N, hc, d), np.uint16)
    dy[P] = dy_val

    def as_dev(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).reshape(c.B, T, hc, d).cuda()

    dh, grads = eg.backward(c.cfg(), c.params, c.dev["ids"], as_dev(hid), as_dev(dy))
    torch.cuda.synchronize()
    got = {k: v.double().cpu().numpy() for k, v in grads.items()}
    got["d_hidden"] = dh.double().cpu().numpy().reshape(N, hc, d)
    ref = sparse_dy_gradients(c, hid, P, dy_val)
    assert np.array_equal(ref["P'"], Pext)
    return c, got, ref


def test_weight_gradient_over_split_chunks(setup):
    c, got, ref = setup
    assert np.abs(ref["d_w_kv"]).max() > 0
    err = normwise(got["d_w_kv"], ref["d_w_kv"])
    assert err <= TOL["bf16"], err


def test_scale_and_tap_gradients(setup):
    c, got, ref = setup
    for k in ("d_gamma_k", "d_gamma_q", "d_conv_w"):
        assert np.abs(ref[k]).max() > 0, k
        err = normwise(got[k], ref[k])
        assert err <= TOL["bf16"], (k, err)


def test_table_gradient_rows(setup):
    c, got, ref = setup
    hit = c.rows_of(ref["P'"])
    err = normwise(got["d_tables"][hit], ref["d_tables"][hit])
    assert err <= TOL["bf16"], err
    rest = np.ones(len(ref["d_tables"]), bool)
    rest[hit] = False
    assert np.count_nonzero(got["d_tables"][rest]) == 0


def test_hidden_gradient(setup):
    c, got, ref = setup
    Pext = ref["P'"]
    err = normwise(got["d_hidden"][Pext], ref["d_hidden"][Pext])
    assert err <= TOL["bf16"], err
    rest = np.ones(c.B * c.T, bool)
    rest[Pext] = False
    assert np.count_nonzero(got["d_hidden"][rest]) == 0
