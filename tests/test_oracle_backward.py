"""Pins of the oracle's gradients (orc_backward), the backward pass of a
training step.  The pages define the forward only; the gradients are its
exact derivatives, so the oracle's chain rule is checked against:
  - torch.autograd in float64 over an independent torch forward (table
    lookup as indexing, torch rms_norm, the page's torch gate activation,
    torch conv1d), gradient by gradient;
  - central finite differences of the oracle's own (pinned) forward at
    sampled entries of every input;
  - the closed form at s = 0 (hidden state zero): no gradient flows through
    the gate's score.
"""
import math

import numpy as np
import pytest
import torch

import engram_synth as S
import oracle as orc

F = torch.nn.functional


def _setup(over=None, seed_dy=5):
    w = S.WORKLOADS["tiny_fp32"].replace(**(over or {}))
    inp = S.Inputs(w)
    o = orc.Oracle.from_workload(w, inp, batch=w.batch, seqlen=w.seqlen)
    args = dict(ids=inp.ids, remap=inp.remap, table=inp.table(), w_kv=inp.wkv(), gamma_k=inp.gamma_k(),
                gamma_q=inp.gamma_q(), conv_w=inp.conv_w(), hidden=inp.hidden())
    dy = np.random.default_rng(seed_dy).standard_normal((w.batch, w.seqlen, w.hc_mult, w.hidden))
    return w, inp, o, args, dy


def _torch_grads(w, inp, o, a, dy):
    T, B, hc, d, K, D = w.seqlen, w.batch, w.hc_mult, w.hidden, w.conv_kernel, w.conv_dilation
    idx = o.hash(a["ids"], remap=a["remap"]).reshape(B * T, -1)
    off = np.concatenate([[0], np.cumsum(inp.primes)[:-1]])
    t64 = lambda x: torch.tensor(np.asarray(x, dtype=np.float64), requires_grad=True)  # noqa: E731
    table, wkv, gk, gq, cw, hid = (t64(a[k]) for k in ("table", "w_kv", "gamma_k", "gamma_q", "conv_w", "hidden"))
    rows = torch.tensor((idx + off[None, :]).ravel())
    e = table.reshape(int(np.sum(inp.primes)), -1)[rows].reshape(B * T, -1)
    kv = e @ wkv.T
    Kk = kv[:, : hc * d].reshape(B * T, hc, d)
    V = kv[:, hc * d:]
    Q = hid.reshape(B * T, hc, d)
    kn = torch.stack([F.rms_norm(Kk[:, h], (d,), gk[h], eps=w.norm_eps) for h in range(hc)], 1)
    qn = torch.stack([F.rms_norm(Q[:, h], (d,), gq[h], eps=w.norm_eps) for h in range(hc)], 1)
    s = (kn * qn).sum(-1) / math.sqrt(d)
    g = (s.abs().clamp_min(w.gate_clamp).sqrt() * s.sign()).sigmoid()
    vg = (g[:, :, None] * V[:, None, :]).reshape(B, T, hc * d)
    conv = F.conv1d(vg.transpose(1, 2), cw.reshape(hc * d, 1, K), groups=hc * d, dilation=D,
                    padding=(K - 1) * D)[:, :, :T].transpose(1, 2)
    y = (vg + conv).reshape(B, T, hc, d)
    (y * torch.tensor(dy)).sum().backward()
    return {"d_table": table.grad.numpy().reshape(-1, w.head_dim), "d_w_kv": wkv.grad.numpy(),
            "d_gamma_k": gk.grad.numpy(), "d_gamma_q": gq.grad.numpy(),
            "d_conv_w": cw.grad.numpy().reshape(hc, d, K), "d_hidden": hid.grad.numpy().reshape(B, T, hc, d)}


@pytest.mark.parametrize("over", [{}, dict(sigma_conv=0.5, sigma_gamma=0.5), dict(hc_mult=3, batch=2, seqlen=40)])
def test_backward_matches_torch_autograd(over):
    w, inp, o, a, dy = _setup(over)
    got = o.backward(dy=dy, **a)
    ref = _torch_grads(w, inp, o, a, dy)
    for k, r in ref.items():
        g = got[k].reshape(r.shape)
        scale = max(np.abs(r).max(), 1e-30)
        assert np.abs(g - r).max() <= 1e-10 * scale, k


def test_backward_matches_finite_differences():
    """d(sum y*dy)/dx at sampled entries of every input, central differences of
    the oracle forward with the inputs stored as float32."""
    w, inp, o, a, dy = _setup()
    got = o.backward(dy=dy, **a)
    loss = lambda aa: float((o.forward(**aa) * dy).sum())  # noqa: E731
    rng = np.random.default_rng(3)
    idx = o.hash(a["ids"], remap=a["remap"])
    off = np.concatenate([[0], np.cumsum(inp.primes)[:-1]])
    used = np.unique((idx.reshape(-1, idx.shape[-1]) + off[None, :]).ravel())
    picks = {"table": [(int(r) * w.head_dim + int(j)) for r, j in zip(rng.choice(used, 6),
                                                                        rng.integers(0, w.head_dim, 6))],
             "w_kv": list(rng.integers(0, a["w_kv"].size, 6)), "gamma_k": list(rng.integers(0, a["gamma_k"].size, 4)),
             "gamma_q": list(rng.integers(0, a["gamma_q"].size, 4)), "conv_w": list(rng.integers(0, a["conv_w"].size, 4)),
             "hidden": list(rng.integers(0, a["hidden"].size, 6))}
    names = {"table": "d_table", "w_kv": "d_w_kv", "gamma_k": "d_gamma_k", "gamma_q": "d_gamma_q",
             "conv_w": "d_conv_w", "hidden": "d_hidden"}
    for arg, flat in picks.items():
        for i in flat:
            base = np.asarray(a[arg], dtype=np.float32)
            x0 = float(base.reshape(-1)[i])
            h = np.float32(max(abs(x0), 1e-2) * 2e-3)
            vals = []
            for sgn in (1, -1):
                pert = base.copy()
                pert.reshape(-1)[i] = np.float32(x0 + sgn * h)
                vals.append((loss({**a, arg: pert}), float(pert.reshape(-1)[i])))
            fd = (vals[0][0] - vals[1][0]) / (vals[0][1] - vals[1][1])
            an = float(got[names[arg]].reshape(-1)[i])
            assert abs(fd - an) <= 1e-4 * max(1.0, abs(an)) + 2e-3 * abs(an), (arg, i, fd, an)


def test_backward_zero_hidden_closed_form():
    """Q = 0 makes s = 0: g = 1/2 everywhere, no gradient flows through the
    score (d hidden = 0, d gamma = 0), and the value path carries dy alone."""
    w, inp, o, a, dy = _setup()
    a = {**a, "hidden": np.zeros_like(a["hidden"])}
    got = o.backward(dy=dy, **a)
    assert np.all(got["d_hidden"] == 0) and np.all(got["d_gamma_k"] == 0) and np.all(got["d_gamma_q"] == 0)
    hc, d = w.hc_mult, w.hidden
    assert np.all(got["d_w_kv"][: hc * d] == 0)          # key rows get nothing
    assert np.abs(got["d_w_kv"][hc * d:]).max() > 0       # value rows do


@pytest.mark.parametrize("name,over", [("tiny_fp32", {}), ("tiny_fp32", dict(hc_mult=3, batch=2, seqlen=40)),
                                       ("b4_t1024", dict(batch=2, seqlen=24, hidden=64, head_dim=8,
                                                         heads_per_order=2, prime_base=101))])
def test_backward_at_matches_dense_backward(name, over):
    """orc_backward_at at every position (sparse rows, each keyed by flat
    position) gives the dense backward's d hidden; its de summed by table row
    gives the dense d_table, its dkv[p] (x) e[p] summed over positions the
    dense d_w_kv, and its summed scale terms the dense d_gamma_k, d_gamma_q
    (all pinned above against autograd)."""
    w = S.WORKLOADS[name].replace(**over)
    inp = S.Inputs(w)
    o = orc.Oracle.from_workload(w, inp, batch=w.batch, seqlen=w.seqlen)
    B, T = w.batch, w.seqlen
    b, t = np.divmod(np.arange(B * T), T)
    hidden, dy = inp.hidden_at(b, t), inp.dy_at(b, t)
    table = inp.table()
    args = dict(ids=inp.ids, remap=inp.remap, table=table, w_kv=inp.wkv(), gamma_k=inp.gamma_k(),
                gamma_q=inp.gamma_q(), conv_w=inp.conv_w())
    dy64 = (dy.astype(np.float32) if w.dtype == "f32" else S.bf16_bits_to_f32(dy)).astype(np.float64)
    dense = o.backward(hidden=hidden.reshape(B, T, w.hc_mult, w.hidden), dy=dy64.reshape(B, T, w.hc_mult, w.hidden),
                       **args)
    # positions in a shuffled order, hidden/dy as sparse rows keyed by position
    pos = np.random.default_rng(0).permutation(B * T)
    keys = np.arange(B * T, dtype=np.int64)
    dh, de, dkv, dgk, dgq = o.backward_at(hidden=hidden, dy=dy, positions=pos, hidden_keys=keys, dy_keys=keys,
                                          want_dkv=True, want_dgamma=True, **args)
    ref_dh = dense["d_hidden"].reshape(B * T, w.hc_mult, w.hidden)[pos]
    assert np.abs(dh - ref_dh).max() <= 1e-12 * np.abs(ref_dh).max()
    idx = o.hash(inp.ids, remap=inp.remap).reshape(B * T, -1)[pos]
    e = o.with_shape(1, len(pos)).gather(table, idx)
    e64 = (e.astype(np.float32) if w.dtype == "f32" else S.bf16_bits_to_f32(e)).astype(np.float64)
    dw = dkv.reshape(len(pos), -1).T @ e64
    assert np.abs(dw - dense["d_w_kv"]).max() <= 1e-12 * np.abs(dense["d_w_kv"]).max()
    for got, ref in ((dgk, dense["d_gamma_k"]), (dgq, dense["d_gamma_q"])):
        assert np.abs(ref).max() > 0
        assert np.abs(got - ref).max() <= 1e-12 * np.abs(ref).max()
    off = np.concatenate([[0], np.cumsum(inp.primes)[:-1]])
    acc = np.zeros_like(dense["d_table"])
    H, Dh = idx.shape[1], w.head_dim
    for h in range(H):
        np.add.at(acc, idx[:, h] + off[h], de[:, h * Dh:(h + 1) * Dh])
    assert np.abs(acc - dense["d_table"]).max() <= 1e-12 * np.abs(dense["d_table"]).max()
    # missing rows are reported, not read
    with pytest.raises(orc.OracleError):
        o.backward_at(hidden=hidden[:5], dy=dy[:5], positions=pos[:1], hidden_keys=keys[:5], dy_keys=keys[:5],
                      **args)


@pytest.mark.parametrize("name,over", [("tiny_fp32", dict(batch=2, seqlen=30, hc_mult=2)),
                                       ("b4_t1024", dict(batch=3, seqlen=40, hidden=64, head_dim=8,
                                                         heads_per_order=2, prime_base=101, hc_mult=2))])
def test_sparse_dy_gradients_equal_dense_backward(name, over):
    """The decomposition the large GPU backward tests rest on
    (cases.sparse_dy_gradients): with dy zero except at a few positions, the
    oracle's per-position gradients at P' = {p - jD} and the zero-tap forward's
    Vg, summed over those positions, give the dense backward's gradients."""
    from cases import Case, sparse_dy_gradients

    c = Case(name, **over)
    w = c.w
    N, hc, d = c.B * c.T, w.hc_mult, w.hidden
    rng = np.random.default_rng(3)
    P = np.unique(np.concatenate([[0, c.T - 1, c.T, N - 1], rng.choice(N, 4, replace=False)]))
    x = rng.standard_normal((len(P), hc, d)).astype(np.float32)
    dy_val = x if w.dtype == "f32" else S.f32_to_bf16_bits(x)
    dy64 = np.zeros((N, hc, d))
    dy64[P] = x if w.dtype == "f32" else S.bf16_bits_to_f32(dy_val)
    hid = c.inp.hidden().reshape(N, hc, d)
    ref = sparse_dy_gradients(c, hid, P, dy_val, chunk=4)
    gk, gq, cw = c.small
    dense = c.orc.backward(ids=c.inp.ids, remap=c.inp.remap, table=c.inp.table(), w_kv=c.wkv, gamma_k=gk,
                           gamma_q=gq, conv_w=cw, hidden=hid.reshape(c.B, c.T, hc, d),
                           dy=dy64.reshape(c.B, c.T, hc, d))
    for k, v in (("d_w_kv", "d_w_kv"), ("d_tables", "d_table"), ("d_gamma_k", "d_gamma_k"),
                 ("d_gamma_q", "d_gamma_q"), ("d_conv_w", "d_conv_w"), ("d_hidden", "d_hidden")):
        r = dense[v].reshape(ref[k].shape)
        assert np.abs(r).max() > 0, k
        assert np.abs(ref[k] - r).max() <= 1e-12 * np.abs(r).max(), k
