"""The C-ABI library on the host (no GPU): it loads, exports every entry point
include/engram.h declares, and validates configurations before any HIP call."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "engram.h")


@pytest.fixture(scope="module")
def eg():
    import hashed_gram_conditional_amd as m

    if not os.path.exists(m.LIB_PATH):
        m.build()
    m.load()
    return m


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(engram_[a-z_]+)\s*\(", text, flags=re.M)


def test_header_declares_the_four_pages_calls():
    names = declared_functions()
    for n in ("engram_hash", "engram_gather", "engram_gate_conv", "engram_forward"):
        assert n in names


def test_library_exports_every_declared_symbol(eg):
    names = declared_functions()
    assert names, "no declarations parsed"
    out = subprocess.run(["nm", "-D", "--defined-only", eg.LIB_PATH], capture_output=True, text=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if l.strip()}
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    assert sorted(names) == sorted(eg.ENTRY_POINTS)
    lib = ctypes.CDLL(eg.LIB_PATH)
    for n in names:
        assert getattr(lib, n) is not None
    # the debug build exports the same interface
    out = subprocess.run(["nm", "-D", "--defined-only", eg.DEBUG_LIB_PATH], capture_output=True, text=True).stdout
    exported_dbg = {l.split()[-1] for l in out.splitlines() if l.strip()}
    assert not [n for n in names if n not in exported_dbg]
    assert eg.load(debug=True).engram_status_string(-1) == b"invalid configuration or argument"


def good(eg, **over):
    kw = dict(batch=2, seqlen=16, vocab=100, orders=[2, 3], heads_per_order=2, head_dim=16, hidden=32, hc_mult=2,
              multipliers=[3, 5, 7], primes=[11, 13, 17, 19], dtype="bf16")
    kw.update(over)
    return eg.EngramConfig.make(**kw)


def test_workspace_and_state_sizes(eg):
    c = good(eg)
    N, E, d, hc = 32, 64, 32, 2
    ws = eg.workspace_size(c)
    assert ws >= N * E * 2 + N * (hc + 1) * d * 2 + N * hc * 4
    assert ws % 256 == 0
    R = 3 * 3 + 1
    assert eg.state_bytes_per_sequence(c) == 2 * 4 + R * d * 2 + R * hc * 4 + 8


@pytest.mark.parametrize("over,status", [
    (dict(orders=[3, 2]), -1), (dict(orders=[0, 3]), -1), (dict(heads_per_order=0), -1),
    (dict(hidden=36), -4), (dict(head_dim=3, heads_per_order=1, primes=[11, 13]), -4),
    (dict(hc_mult=0), -1), (dict(hc_mult=17), -1), (dict(conv_kernel=9), -1), (dict(conv_dilation=0), -1),
    (dict(primes=[11, 0, 17, 19]), -1), (dict(primes=[11, 13, 17, 2**31]), -1), (dict(vocab=0), -1),
    (dict(batch=-1), -1), (dict(norm_eps=-1.0), -1),
])
def test_invalid_configs_are_rejected_on_the_host(eg, over, status):
    c = good(eg, **over)
    assert eg.workspace_size(c) == 0
    lib = eg.load()
    P = ctypes.c_void_p
    prm = eg._Params(P(16), P(16), P(16), P(16), P(16), P(16))
    # validation fails before any pointer is touched or kernel enqueued
    rc = lib.engram_hash(ctypes.byref(c), ctypes.byref(prm), P(16), None, P(16), None)
    assert rc == status
    rc = lib.engram_forward(ctypes.byref(c), ctypes.byref(prm), P(16), P(16), None, P(16), P(256), 1 << 30, None)
    assert rc == status


def test_forward_rejects_short_workspace_and_null_pointers(eg):
    c = good(eg)
    lib = eg.load()
    P = ctypes.c_void_p
    prm = eg._Params(P(16), P(16), P(16), P(16), P(16), P(16))
    ws = eg.workspace_size(c)
    assert lib.engram_forward(ctypes.byref(c), ctypes.byref(prm), P(16), P(16), None, P(16), P(256), ws - 1,
                              None) == -2
    assert lib.engram_forward(ctypes.byref(c), ctypes.byref(prm), None, P(16), None, P(16), P(256), ws, None) == -1
    prm_bad = eg._Params(P(16), None, P(16), P(16), P(16), P(16))
    assert lib.engram_forward(ctypes.byref(c), ctypes.byref(prm_bad), P(16), P(16), None, P(16), P(256), ws,
                              None) == -1
    # misaligned device pointers
    assert lib.engram_forward(ctypes.byref(c), ctypes.byref(prm), P(16), P(18), None, P(16), P(256), ws, None) == -1
    # every parameter array but remap is 16-byte aligned (the conv taps are read 8 or 16 bytes at a time)
    for i in range(1, 6):
        args = [P(16)] * 6
        args[i] = P(16 + 4)
        bad = eg._Params(*args)
        assert lib.engram_forward(ctypes.byref(c), ctypes.byref(bad), P(16), P(16), None, P(16), P(256), ws,
                                  None) == -1, i


def test_empty_calls_succeed_without_launching(eg):
    lib = eg.load()
    P = ctypes.c_void_p
    prm = eg._Params(P(16), P(16), P(16), P(16), P(16), P(16))
    for B, T in ((0, 16), (2, 0)):
        c = good(eg, batch=B, seqlen=T)
        assert lib.engram_hash(ctypes.byref(c), ctypes.byref(prm), None, None, None, None) == 0
        assert lib.engram_forward(ctypes.byref(c), ctypes.byref(prm), None, None, None, None, None, 0, None) == 0


def test_status_strings_and_kernel_names(eg):
    lib = eg.load()
    assert lib.engram_status_string(-2) == b"workspace too small"
    assert eg.kernel_names(good(eg), with_state=True) == ["hash_gather", "project_gemm", "gate", "short_conv",
                                                         "advance_state"]
    # every plan: stored projections, fused, split, decode tail
    fused = dict(hidden=2560, hc_mult=4, orders=[2, 3], heads_per_order=8, head_dim=64,
                 primes=list(range(1, 17)), multipliers=[3, 5, 7])
    assert eg.kernel_names(good(eg, batch=16, seqlen=256, **fused)) == ["hash_gather", "project_gate_gemm",
                                                                       "gate_finalize", "short_conv"]
    assert eg.kernel_names(good(eg, batch=4, seqlen=1024, **dict(fused, hidden=1024))) == [
        "hash_gather", "project_gate_gemm", "project_value_gemm", "short_conv"]
    assert eg.kernel_names(good(eg, batch=256, seqlen=1, **fused), with_state=True) == [
        "hash_gather", "project_gate_gemm", "decode_tail"]
    assert eg.kernel_names(good(eg, batch=256, seqlen=1, **fused), with_state=False) == [
        "hash_gather", "project_gate_gemm", "gate_finalize", "short_conv"]


def test_forward_gathered_validates_on_the_host(eg):
    """engram_forward_gathered: the rows must be given (16-byte aligned); the
    tables and (without a state) the ids are not needed.  A short workspace is
    reported only once everything else passed, so -2 shows the rest was accepted."""
    c = good(eg)
    lib = eg.load()
    P = ctypes.c_void_p
    ws = eg.workspace_size(c)
    no_tables = eg._Params(P(16), None, P(16), P(16), P(16), P(16))
    f = lib.engram_forward_gathered
    assert f(ctypes.byref(c), ctypes.byref(no_tables), None, P(16), P(16), None, P(16), P(256), ws - 1, None) == -2
    assert f(ctypes.byref(c), ctypes.byref(no_tables), None, None, P(16), None, P(16), P(256), ws, None) == -1
    assert f(ctypes.byref(c), ctypes.byref(no_tables), None, P(24), P(16), None, P(16), P(256), ws, None) == -1
    no_w = eg._Params(P(16), P(16), None, P(16), P(16), P(16))
    assert f(ctypes.byref(c), ctypes.byref(no_w), None, P(16), P(16), None, P(16), P(256), ws, None) == -1
    empty = good(eg, batch=0)
    assert f(ctypes.byref(empty), ctypes.byref(no_tables), None, None, None, None, None, None, 0, None) == 0


@pytest.mark.parametrize("name,over", [("tiny_fp32", {}),
                                       ("b4_t1024", dict(batch=2, seqlen=300, prime_base=4001))])
def test_host_gather_matches_oracle(eg, name, over):
    """engram_gather_host (host memory, no GPU): every gathered row equals the
    oracle's, bit for bit, on 1 and on several threads; indices out of range
    are clamped like the device gather."""
    import numpy as np

    from cases import Case

    c = Case(name, **over)
    cfg = c.cfg()
    N = c.B * c.T
    table = np.ascontiguousarray(c.inp.table())
    idx = np.ascontiguousarray(c.idx.astype(np.int32))
    ref = c.e_at(np.arange(N)).reshape(N, -1)
    for threads in (1, 3, 0):
        out = np.zeros_like(ref)
        eg.engram_gather_host(cfg, table, idx, out, n_threads=threads)
        assert np.array_equal(out, ref)
    bad = idx.copy()
    bad.reshape(-1)[:5] = [-1, 2**30, -5, 2**31 - 1, 0]
    out = np.zeros_like(ref)
    eg.engram_gather_host(cfg, table, bad, out)
    H = idx.shape[-1]
    p = np.asarray(c.inp.primes, dtype=np.int64)
    clamped = np.clip(bad.reshape(N, H).astype(np.int64), 0, p[None, :] - 1)
    off = np.concatenate([[0], np.cumsum(p)[:-1]])
    rows = table.reshape(int(p.sum()), -1)[(clamped + off[None, :]).ravel()].reshape(N, -1)
    assert np.array_equal(out, rows)


def test_hash_layers_validates_on_the_host(eg):
    c = good(eg)
    lib = eg.load()
    P = ctypes.c_void_p
    prm = eg._Params(P(16), P(16), P(16), P(16), P(16), P(16))
    mult = (ctypes.c_int64 * (16 * 8))(*range(1, 129))
    f = lib.engram_hash_layers
    assert f(ctypes.byref(c), ctypes.byref(prm), P(16), None, mult, 0, P(16), None) == -1
    assert f(ctypes.byref(c), ctypes.byref(prm), P(16), None, mult, 17, P(16), None) == -1
    assert f(ctypes.byref(c), ctypes.byref(prm), P(16), None, None, 2, P(16), None) == -1
    assert f(ctypes.byref(c), ctypes.byref(prm), None, None, mult, 2, P(16), None) == -1
    empty = good(eg, batch=0)
    assert f(ctypes.byref(empty), ctypes.byref(prm), None, None, mult, 2, None, None) == 0


def test_backward_validates_on_the_host(eg):
    """engram_backward: every gradient and input pointer is required (hidden,
    dy, d hidden 16-byte aligned); a short workspace is reported only once
    the rest passed; an empty batch succeeds with nothing launched."""
    c = good(eg)
    lib = eg.load()
    P = ctypes.c_void_p
    prm = eg._Params(P(16), P(16), P(16), P(16), P(16), P(16))
    ws = lib.engram_backward_workspace_size(ctypes.byref(c))
    N, E, O = 32, 64, 3 * 32
    assert ws >= N * E * (2 + 4) + N * O * 2 * 2 + N * 2 * 16
    assert lib.engram_backward_workspace_size(ctypes.byref(good(eg, hc_mult=0))) == 0
    f = lib.engram_backward
    ok = [P(16), P(16), P(16), P(16), P(16), P(16), P(16), P(16), P(16)]
    assert f(ctypes.byref(c), ctypes.byref(prm), *ok, P(256), ws - 1, None) == -2
    for i in range(len(ok)):
        args = list(ok)
        args[i] = None
        assert f(ctypes.byref(c), ctypes.byref(prm), *args, P(256), ws, None) == -1, i
    args = list(ok)
    args[1] = P(24)
    assert f(ctypes.byref(c), ctypes.byref(prm), *args, P(256), ws, None) == -1
    assert f(ctypes.byref(c), ctypes.byref(prm), *ok, None, ws, None) == -1
    empty = good(eg, batch=0)
    assert f(ctypes.byref(empty), ctypes.byref(prm), *([None] * 9), None, 0, None) == 0


def test_forward_train_and_backward_saved_validate_on_the_host(eg):
    """engram_forward_train needs ids, hidden, out and a backward-sized
    workspace; engram_backward_saved needs no ids and no tables."""
    c = good(eg)
    lib = eg.load()
    P = ctypes.c_void_p
    prm = eg._Params(P(16), P(16), P(16), P(16), P(16), P(16))
    no_tables = eg._Params(P(16), None, P(16), P(16), P(16), P(16))
    ws = lib.engram_backward_workspace_size(ctypes.byref(c))
    f = lib.engram_forward_train
    assert f(ctypes.byref(c), ctypes.byref(prm), P(16), P(16), P(16), P(256), ws - 1, None) == -2
    assert f(ctypes.byref(c), ctypes.byref(no_tables), P(16), P(16), P(16), P(256), ws, None) == -1
    assert f(ctypes.byref(c), ctypes.byref(prm), None, P(16), P(16), P(256), ws, None) == -1
    assert f(ctypes.byref(c), ctypes.byref(prm), P(16), P(24), P(16), P(256), ws, None) == -1
    assert f(ctypes.byref(c), ctypes.byref(prm), P(16), P(16), P(16), P(128), ws, None) == -1
    g = lib.engram_backward_saved
    ok = [P(16)] * 8
    assert g(ctypes.byref(c), ctypes.byref(no_tables), *ok, P(256), ws - 1, None) == -2
    for i in range(len(ok)):
        args = list(ok)
        args[i] = None
        assert g(ctypes.byref(c), ctypes.byref(no_tables), *args, P(256), ws, None) == -1, i
    no_w = eg._Params(P(16), None, None, P(16), P(16), P(16))
    assert g(ctypes.byref(c), ctypes.byref(no_w), *ok, P(256), ws, None) == -1
    empty = good(eg, batch=0)
    assert f(ctypes.byref(empty), ctypes.byref(prm), None, None, None, None, 0, None) == 0
    assert g(ctypes.byref(empty), ctypes.byref(no_tables), *([None] * 8), None, 0, None) == 0
