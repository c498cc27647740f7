"""Tables in host memory (architecture walk-through, yaoyuxiang.cn/news/830577,
section 4.4, inference: the tables can live in host memory because the hash
depends only on the token ids, so the rows a layer needs are known, and can be
fetched, before the layer runs).

The tables go to pinned host memory mapped into the device; the gather then
reads them over the host link.  Each flow is checked against the oracle --
indices and gathered rows bit for bit, outputs within the bf16 bar at the
first positions of a sequence and at seeded positions -- and bit for bit against
the same calls with the tables in HBM:
  - the whole forward reading host-resident tables;
  - the prefetch flow: hash + gather from host tables on a side stream, then
    the forward on the gathered rows (engram_forward_gathered);
  - the same flow across a chunked prefill and decode steps with a state;
  - the host-thread row copy (engram_gather_host) plus a DMA copy.
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


@pytest.fixture(scope="module")
def c4():
    return Case("b4_t1024")


@pytest.fixture(scope="module")
def host_params(eg, c4):
    d = c4.dev
    t = d["tables"]
    host = eg.alloc_mapped_host(t.numel() * t.element_size())
    host.copy_from(t)
    p = eg.Params(remap=d["remap"], tables=host, w_kv=d["w_kv"], gamma_k=d["gamma_k"], gamma_q=d["gamma_q"],
                  conv_w=d["conv_w"])
    yield p
    torch.cuda.synchronize()
    host.free()


@pytest.fixture(scope="module")
def y_ref(c4):
    """The oracle's outputs at the first 16 positions, the last one and 256
    seeded ones."""
    pos = c4.sample_positions(256, seed=31)
    return pos, c4.y_at_many(pos)


def _check_y(c4, y, y_ref):
    pos, ref = y_ref
    got = to_f64(y).reshape(c4.B * c4.T, c4.w.hc_mult, c4.w.hidden)[pos]
    err = normwise(got, ref)
    assert err <= TOL["bf16"], err


def _check_rows(c4, e):
    from engram_synth.device import storage_numpy

    N = c4.B * c4.T
    got = storage_numpy(e.cpu() if e.is_cuda else e).reshape(N, -1)
    assert np.array_equal(got, c4.e_at(np.arange(N)))


def test_forward_with_host_tables_is_bit_equal(eg, c4, host_params, y_ref):
    d = c4.dev
    y_dev = eg.forward(c4.cfg(), c4.params, d["ids"], d["hidden"])
    y_host = eg.forward(c4.cfg(), host_params, d["ids"], d["hidden"])
    torch.cuda.synchronize()
    assert torch.equal(y_dev, y_host)
    _check_y(c4, y_host, y_ref)


def test_prefetch_then_gathered_forward_is_bit_equal(eg, c4, host_params, y_ref):
    d = c4.dev
    cfg = c4.cfg()
    y_dev = eg.forward(cfg, c4.params, d["ids"], d["hidden"])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        idx = eg.engram_hash(cfg, host_params, d["ids"], stream=side)
        e = eg.engram_gather(cfg, host_params, idx, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    no_tables = eg.Params(remap=d["remap"], tables=None, w_kv=d["w_kv"], gamma_k=d["gamma_k"], gamma_q=d["gamma_q"],
                          conv_w=d["conv_w"])
    y = eg.forward_gathered(cfg, no_tables, e, d["hidden"])
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy().astype(np.int64), c4.idx)
    _check_rows(c4, e)
    _check_y(c4, y, y_ref)
    assert torch.equal(y, y_dev)


def test_prefetch_flow_with_state(eg, c4, host_params):
    """Chunked prefill then single-token steps: hash (reading the state's token
    history) and gather ahead, then the gathered forward advancing the state,
    equal engram_forward with the same state sequence; the indices and rows of
    each chunk equal the oracle's, and the outputs of the whole first sequence
    and of 128 seeded positions the oracle's."""
    from engram_synth.device import storage_numpy

    d = c4.dev
    B = c4.B
    st_ref, st = eg.State(c4.cfg(), B), eg.State(c4.cfg(), B)
    t0 = 0
    ys = []
    for L in (300, 1, 1, 50, 1):
        ids = d["ids"][:, t0:t0 + L].contiguous()
        hid = d["hidden"][:, t0:t0 + L].contiguous()
        cfg = c4.cfg(B, L)
        ref = eg.forward(cfg, c4.params, ids, hid, state=st_ref)
        idx = eg.engram_hash(cfg, host_params, ids, state=st)
        e = eg.engram_gather(cfg, host_params, idx)
        y = eg.forward_gathered(cfg, host_params, e, hid, ids=ids, state=st)
        torch.cuda.synchronize()
        assert torch.equal(y, ref), (t0, L)
        assert np.array_equal(idx.cpu().numpy().astype(np.int64), c4.idx[:, t0:t0 + L]), (t0, L)
        pos = (np.arange(B)[:, None] * c4.T + np.arange(t0, t0 + L)[None, :]).ravel()
        assert np.array_equal(storage_numpy(e).reshape(B * L, -1), c4.e_at(pos)), (t0, L)
        ys.append(to_f64(y))
        t0 += L
    y = np.concatenate(ys, axis=1)                 # [B][t0][hc][d]
    rng = np.random.default_rng(8)
    pos = np.unique(np.concatenate([np.arange(t0), rng.choice(B * t0, 128, replace=False)]))
    b, t = np.divmod(pos, t0)
    err = normwise(y[b, t], c4.y_at_many(b * c4.T + t))
    assert err <= TOL["bf16"], err
    assert torch.equal(st.n_past, st_ref.n_past)
    assert torch.equal(st.v_ring, st_ref.v_ring) and torch.equal(st.tok_ring, st_ref.tok_ring)


def test_host_gather_and_dma_flow_is_bit_equal(eg, c4, host_params, y_ref):
    """The flow that keeps the lookup off the GPU's compute units: hash on the
    GPU, indices copied to host memory, rows copied on the host
    (engram_gather_host), rows copied to the device, gathered forward."""
    d = c4.dev
    cfg = c4.cfg()
    y_dev = eg.forward(cfg, c4.params, d["ids"], d["hidden"])
    idx = eg.engram_hash(cfg, c4.params, d["ids"])
    idx_h = torch.empty(idx.shape, dtype=torch.int32, pin_memory=True)
    idx_h.copy_(idx)
    e_h = torch.empty((c4.B, c4.T, cfg.emb_dim), dtype=torch.bfloat16, pin_memory=True)
    eg.engram_gather_host(cfg, host_params.tables, idx_h, e_h)
    e = e_h.to("cuda", non_blocking=True)
    y = eg.forward_gathered(cfg, host_params, e, d["hidden"])
    torch.cuda.synchronize()
    _check_rows(c4, e_h)
    _check_y(c4, y, y_ref)
    assert torch.equal(y, y_dev)
