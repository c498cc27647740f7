"""engram_forward_noalloc (the forward for callers that cannot allocate: its
workspace is a device array inside the library) against engram_forward with
a caller workspace: bit-equal outputs on two calls in a row, the second with
fewer tokens, with and without a decode state; and the size limit."""
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def eg():
    import hashed_gram_conditional_amd as m

    m.load()
    return m


def _case(name, **over):
    from cases import Case

    return Case(name, **over)


def test_noalloc_equals_forward_on_two_calls(eg):
    c = _case("b4_t1024")
    d = c.dev
    for B, T in ((4, 1024), (3, 200)):           # the second call smaller
        cfg = c.cfg(B, T)
        ids = d["ids"][:B, :T].contiguous()
        hid = d["hidden"][:B, :T].contiguous()
        ref = eg.forward(cfg, c.params, ids, hid)
        got = eg.forward_noalloc(cfg, c.params, ids, hid)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), (B, T)


def test_noalloc_with_state_equals_forward(eg):
    """A chunked prefill and decode steps through the no-allocation entry point
    give engram_forward's outputs and states bit for bit."""
    c = _case("decode_b256", batch=64)
    d = c.dev
    P = c.w.decode_prompt
    st_ref, st = eg.State(c.cfg(64, 1), 64), eg.State(c.cfg(64, 1), 64)
    t0 = 0
    for L in (P, 1, 1, 1):
        cfg = c.cfg(64, L)
        ids = d["ids"][:, t0:t0 + L].contiguous()
        hid = d["hidden"][:, t0:t0 + L].contiguous()
        ref = eg.forward(cfg, c.params, ids, hid, state=st_ref)
        got = eg.forward_noalloc(cfg, c.params, ids, hid, state=st)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), (t0, L)
        t0 += L
    for a, b in ((st.tok_ring, st_ref.tok_ring), (st.v_ring, st_ref.v_ring), (st.g_ring, st_ref.g_ring),
                 (st.n_past, st_ref.n_past)):
        assert torch.equal(a, b)


def test_noalloc_rejects_a_workspace_beyond_its_array(eg):
    """32768 tokens at hidden 1024 need more workspace than the array holds:
    ENGRAM_ENOMEM, nothing enqueued."""
    import hashed_gram_conditional_amd as m

    c = _case("b4_t1024")
    cfg = c.cfg(32, 1024)
    assert eg.workspace_size(cfg) > m.NOALLOC_MAX_BYTES >= eg.workspace_size(c.cfg())
    ids = torch.zeros((32, 1024), dtype=torch.int32, device="cuda")
    out = torch.zeros((1, 1, c.w.hc_mult, c.w.hidden), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(m.EngramError) as ei:
        eg.forward_noalloc(cfg, c.params, ids, out, out=out)
    assert ei.value.status == -2
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(out)) == 0
