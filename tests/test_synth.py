"""Seeded input generator checks (CPU only)."""
import numpy as np
import pytest

import engram_synth as S


def test_mix64_matches_published_splitmix64_output():
    # SplitMix64 from state 0: the first output is mix64(0 + golden gamma)
    assert int(S.mix64(np.array([0x9E3779B97F4A7C15], np.uint64))[0]) == 0xE220A8397B1DCDAF


def test_streams_are_reproducible_and_random_access():
    a = S.stream_z(7, 3, np.arange(1000))
    b = S.stream_z(7, 3, np.arange(500, 1000))
    assert np.array_equal(a[500:], b)
    assert not np.array_equal(a, S.stream_z(7, 4, np.arange(1000)))
    assert len(np.unique(a)) == 1000


def test_ih4_moments_and_bf16_rounding():
    v = S.ih4_values(1, 6, np.arange(200000), 0.02, 0.0)
    assert abs(v.mean()) < 2e-4 and abs(v.std() - 0.02) < 3e-4
    assert np.abs(v).max() <= 0.02 * np.sqrt(3) * 2 + 1e-6
    x = np.array([1.0, 1.00390625, 1.01171875, -3.5, 1.0 + 2**-8 + 2**-20], np.float32)
    # ties to even at 1 + 2^-8 (rounds down to 1.0) and 1 + 3*2^-8 (rounds up); above the tie rounds up
    got = S.bf16_bits_to_f32(S.f32_to_bf16_bits(x))
    assert got.tolist() == [1.0, 1.0, 1.015625, -3.5, 1.0078125]


def test_primes_and_workload_shapes():
    assert S.primes_from(1009, 4) == [1009, 1013, 1019, 1021]
    w = S.WORKLOADS["b8_t4096"]
    p = w.primes
    assert len(p) == 16 and len(set(p)) == 16 and min(p) >= 1500000
    assert w.vocab_c == 99545 and w.emb_dim == 1024 and w.conv_dilation == 3
    w5 = S.WORKLOADS["b1_t32768"]
    assert w5.n_heads == 24 and w5.conv_dilation == 4 and w5.table_rows > 480_000_000


def test_remap_is_surjective_and_tokens_are_zipf():
    w = S.WORKLOADS["b4_t1024"]
    inp = S.Inputs(w)
    assert inp.remap.min() == 0 and inp.remap.max() == w.vocab_c - 1
    assert len(np.unique(inp.remap)) == w.vocab_c
    ids = inp.ids
    assert ids.shape == (4, 1024) and ids.min() >= 0 and ids.max() < w.vocab
    counts = np.sort(np.bincount(ids.ravel(), minlength=w.vocab))[::-1]
    h = (np.arange(1, w.vocab + 1, dtype=np.float64) ** -1.1).sum()
    assert abs(counts[0] / ids.size - 1 / h) < 0.03
    assert counts[0] > 2 * counts[3]


def test_multipliers_are_odd_and_positive():
    m = S.make_multipliers(5, 4)
    assert (m % 2 == 1).all() and (m > 0).all()


def test_hidden_at_matches_dense():
    w = S.WORKLOADS["tiny_fp32"]
    inp = S.Inputs(w)
    full = inp.hidden()
    assert np.array_equal(inp.hidden_at([0, 0], [5, 63]), full[0, [5, 63]])
    assert np.array_equal(inp.table_rows([3, 4000]), inp.table()[[3, 4000]])
