"""GPU parity of det_index_add against the CPU oracle (bitwise), chunk-size
coverage, padding/bad ids, replay under load and the atomic arm."""
import numpy as np
import pytest

import deterministic_gradient_reductions_amd as dg
import workloads as W
from oracle import index_add as oi
from tests.gpu_util import SideLoad, assert_bitwise, dev_bf16, dev_f32, dev_i32, host, note, rel_l2

pytestmark = pytest.mark.gpu


def run(ids, src, out0, L=None, atomic=False, ws=None, src_pad=0):
    import torch
    P, D = src.shape
    dev_src = dev_f32 if src.dtype == np.float32 else dev_bf16  # float32 values or bf16 bits
    if src_pad:
        sb = np.zeros((P, D + src_pad), src.dtype); sb[:, :D] = src
        s = dev_src(sb)[:, :D]
    else:
        s = dev_src(src)
    o = dev_f32(out0)
    i = dev_i32(ids)
    torch.cuda.synchronize()
    dg.det_index_add(o, i, s, cfg=None if L is None else dg.IndexAddCfg(L), atomic=atomic, ws=ws)
    return host(o)


def small(P, n_rows, dim, seed, pad=0.05, out_init="normal", dtype="bf16"):
    ids = W.zipf_ids(P, n_rows, 1.1, pad, seed)
    rng = np.random.default_rng(seed + 100)
    src = rng.standard_normal((P, dim)).astype(np.float32) * np.float32(0.02)
    if dtype == "bf16":
        src = W.bf16_bits(src)
    out0 = rng.standard_normal((n_rows, dim)).astype(np.float32) if out_init == "normal" else \
        np.zeros((n_rows, dim), np.float32)
    return ids, src, out0


@pytest.mark.parametrize("P,n_rows,dim", [(5000, 64, 128), (20000, 1000, 128), (3000, 7, 8), (9000, 300, 64),
                                          (4097, 8192, 128), (1, 1, 16), (12345, 513, 512), (8192, 16384, 24),
                                          (20000, 5, 40), (30000, 3, 48)])
@pytest.mark.parametrize("L", [1, 7, 256, 512, 1024])
def test_parity_small(P, n_rows, dim, L):
    note("index_add P=%d rows=%d dim=%d L=%d" % (P, n_rows, dim, L))
    ids, src, out0 = small(P, n_rows, dim, seed=P % 97)
    got = run(ids, src, out0, L)
    assert_bitwise(got, oi.index_add(out0, ids, src, L), "index_add")


def test_bad_ids_dropped_and_counted():
    ids, src, out0 = small(6000, 100, 128, seed=3)
    ids = ids.copy()
    ids[::50] = 100       # just out of range
    ids[7::333] = -7      # negative, not padding
    ids[3::1000] = 2 ** 30
    n_bad = int(np.sum((ids != -1) & ((ids < 0) | (ids >= 100))))
    ws = dg.Workspace(dg.det_index_add_workspace_size(6000, 128, 100, dg.IndexAddCfg(64)))
    got = run(ids, src, out0, 64, ws=ws)
    assert_bitwise(got, oi.index_add(out0, ids, src, 64), "index_add bad ids")
    assert dg.det_index_add_bad_ids(ws) == n_bad
    # the counter resets: a clean call reports 0
    ok = np.where((ids >= 0) & (ids < 100), ids, -1).astype(np.int32)
    run(ok, src, out0, 64, ws=ws)
    assert dg.det_index_add_bad_ids(ws) == 0


def test_all_padding_and_row_stride():
    ids, src, out0 = small(3000, 50, 128, seed=4)
    got = run(np.full(3000, -1, np.int32), src, out0, 64)
    assert_bitwise(got, out0, "all padding")
    got = run(ids, src, out0, 32, src_pad=8)
    assert_bitwise(got, oi.index_add(out0, ids, src, 32), "row stride")


def test_literal_sequential_order_with_long_chunks():
    """chunk_rows >= the longest run reproduces out[id] += src in stable sorted order from +0."""
    from oracle import brute
    ids, src, out0 = small(2000, 20, 16, seed=5, out_init="zero")
    got = run(ids, src, out0, 65536)
    assert_bitwise(got, brute.literal_sequential_index_add(out0, ids, src), "literal")


@pytest.fixture(scope="module")
def full_inputs():
    return W.index_add_inputs(seed=3, out_init="normal")


@pytest.mark.parametrize("L", [64, 128, 256, 512, 1024])
def test_full_size_parity(full_inputs, L):
    """4096 x 512 Zipf ids -> 8192 x 128 at every chunk length the gather instantiates (L <= 256 one wave of
    rows per chunk; 257..512 and 513..1024 the longer position-register variants)."""
    inp = full_inputs
    note("index_add full size 4096x512 ids -> 8192x128, L=%d" % L)
    got = run(inp.ids, inp.src, inp.out0, L)
    want = oi.index_add(inp.out0, inp.ids, inp.src, L)
    assert_bitwise(got, want, "index_add full L=%d" % L)


def test_replay_under_load_and_atomic_arm():
    import torch
    ids, src, out0 = small(600_000, 8192, 128, seed=6)
    want = oi.index_add(out0, ids, src, 256)
    i, s, o0 = dev_i32(ids), dev_bf16(src), dev_f32(out0)
    ws = dg.Workspace(dg.det_index_add_workspace_size(600_000, 128, 8192))
    load = SideLoad()
    atoms = []
    for r in range(20):
        o = o0.clone()
        load.kick()
        dg.det_index_add(o, i, s, cfg=dg.IndexAddCfg(256), ws=ws)
        assert_bitwise(host(o), want, "replay %d" % r)
        a = o0.clone()
        load.kick()
        dg.det_index_add(a, i, s, atomic=True)
        atoms.append(host(a))
    load.wait()
    for a in atoms:
        assert rel_l2(a - out0, want - out0) <= 1e-5
    distinct = len({a.tobytes() for a in atoms})
    note("index_add atomic arm: %d distinct patterns in 20 runs" % distinct)
    assert distinct > 1, "the atomic arm is bit-stable here, so the replay check could not fail"


def test_exact_integer_sources():
    rng = np.random.default_rng(9)
    P, n_rows, D = 100_000, 500, 128
    ids = W.zipf_ids(P, n_rows, 1.1, 0.05, 9)
    k = rng.integers(-8, 9, (P, D))
    src = W.bf16_bits((k / 256.0).astype(np.float32))
    out0 = np.zeros((n_rows, D), np.float32)
    exact = np.zeros((n_rows, D), np.int64)
    ok = ids >= 0
    np.add.at(exact, ids[ok], k[ok])
    for atomic in (False, True):
        got = run(ids, src, out0, 128, atomic=atomic)
        assert np.array_equal((got * 256).astype(np.int64), exact)


@pytest.mark.parametrize("P,n_rows,dim,L", [(5000, 64, 128, 7), (20000, 1000, 128, 256), (3000, 7, 8, 1),
                                            (9000, 300, 64, 256), (12345, 513, 512, 64), (8192, 16384, 24, 7),
                                            (4000, 50, 128, 65536)])
def test_f32_sources(P, n_rows, dim, L):
    """float32 source rows (the lane-group gather and the long-chunk gather), bitwise."""
    note("index_add f32 src P=%d rows=%d dim=%d L=%d" % (P, n_rows, dim, L))
    ids, src, out0 = small(P, n_rows, dim, seed=P % 89, dtype="f32")
    got = run(ids, src, out0, L)
    assert_bitwise(got, oi.index_add(out0, ids, src, L), "index_add f32")
    got = run(ids, src, out0, L, src_pad=8)
    assert_bitwise(got, oi.index_add(out0, ids, src, L), "index_add f32 row stride")


def test_f32_sources_full_size_and_atomic_arm():
    inp = W.index_add_inputs(seed=3, out_init="normal", dtype="f32")
    note("index_add full size with float32 sources")
    want = oi.index_add(inp.out0, inp.ids, inp.src, 256)
    assert_bitwise(run(inp.ids, inp.src, inp.out0, 256), want, "index_add f32 full")
    a = run(inp.ids, inp.src, inp.out0, atomic=True)
    assert rel_l2(a - inp.out0, want - inp.out0) <= 1e-5
