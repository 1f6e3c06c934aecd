"""GPU parity of det_indexer_dk (the fused sparse-indexer dK) against the CPU
oracle (bitwise), its equality with det_index_add on the explicit float32
source rows, replay under load and the atomic arm."""
import numpy as np
import pytest

import deterministic_gradient_reductions_amd as dg
import workloads as W
from oracle import indexer_dk as ok
from tests.gpu_util import SideLoad, assert_bitwise, dev_bf16, dev_f32, dev_i32, host, note, rel_l2

pytestmark = pytest.mark.gpu


def run(inp, L=None, atomic=False, ws=None, q_pad=0, dk_pad=0, dk0=None):
    import torch
    Q, D = inp.q.shape
    if q_pad:
        qb = np.zeros((Q, D + q_pad), np.uint16); qb[:, :D] = inp.q
        q = dev_bf16(qb)[:, :D]
    else:
        q = dev_bf16(inp.q)
    base = inp.dk0 if dk0 is None else dk0
    if dk_pad:
        db = np.zeros((base.shape[0], D + dk_pad), np.float32); db[:, :D] = base
        dk = dev_f32(db)[:, :D]
    else:
        dk = dev_f32(base)
    torch.cuda.synchronize()
    dg.det_indexer_dk(dk, dev_i32(inp.ids), dev_f32(inp.predict), dev_f32(inp.target), q, inp.scale,
                      cfg=None if L is None else dg.IndexAddCfg(L), atomic=atomic, ws=ws)
    return host(dk)


def want(inp, L=256, dk0=None):
    return ok.indexer_dk(inp.dk0 if dk0 is None else dk0, inp.ids, inp.predict, inp.target, inp.q, inp.scale, L)


@pytest.mark.parametrize("Q,K,n_rows,dim", [(64, 512, 1000, 128), (300, 64, 40, 256), (17, 1000, 8192, 128),
                                            (129, 33, 5, 512), (1, 7, 3, 128), (2048, 128, 16384, 128)])
@pytest.mark.parametrize("L", [1, 7, 256, 1024])
def test_parity_small(Q, K, n_rows, dim, L):
    note("indexer_dk Q=%d K=%d rows=%d dim=%d L=%d" % (Q, K, n_rows, dim, L))
    inp = W.indexer_dk_inputs(Q=Q, K=K, n_rows=n_rows, dim=dim, seed=Q % 31, out_init="normal")
    assert_bitwise(run(inp, L), want(inp, L), "indexer_dk")


@pytest.fixture(scope="module")
def full():
    return W.indexer_dk_inputs(seed=8, out_init="normal")


@pytest.mark.parametrize("L", [64, 256, 1024])
def test_full_size_parity(full, L):
    note("indexer_dk full size 4096x512 -> 8192x128, L=%d" % L)
    assert_bitwise(run(full, L), want(full, L), "indexer_dk full L=%d" % L)


def test_equals_index_add_of_the_explicit_source_rows(full):
    """The fused call and det_index_add on the float32 rows c * q (built by the oracle) give the same bits."""
    import torch
    coef = ok.coefficients(full.ids, full.predict, full.target, full.n_rows, full.scale)
    src = ok.source_rows(coef, full.q)
    o = dev_f32(full.dk0)
    torch.cuda.synchronize()
    dg.det_index_add(o, dev_i32(full.ids.reshape(-1)), dev_f32(src), cfg=dg.IndexAddCfg(256))
    assert_bitwise(run(full, 256), host(o), "fused vs unfused")


def test_exact_dyadic_inputs_and_strides():
    # K = 16: |src| <= 8 in units of 2^-9, at most ~600 rows per key: every partial sum in any order is exact
    inp = W.indexer_dk_inputs(Q=256, K=16, n_rows=300, dim=128, seed=4, integer=True)
    ok_rows = np.bincount(inp.ids[inp.ids >= 0], minlength=300).max()
    assert ok_rows * 8 * 512 < 2 ** 24
    got = run(inp, 16, q_pad=8, dk_pad=4)
    assert_bitwise(got, want(inp, 16), "exact")
    # every partial sum is exact here, so the atomic arm gives the same bits
    assert_bitwise(run(inp, atomic=True), want(inp, 16), "exact atomic")


def test_bad_ids_dropped_and_counted():
    inp = W.indexer_dk_inputs(Q=128, K=96, n_rows=200, dim=128, seed=5, out_init="normal")
    ids = inp.ids.copy()
    ids[::7, 3] = 200
    ids[5, :] = -3
    n_bad = int(np.sum((ids != -1) & ((ids < 0) | (ids >= 200))))
    inp = W.IndexerDkInputs(inp.n_rows, inp.dim, ids, inp.predict, inp.target, inp.q, inp.scale, inp.dk0)
    ws = dg.Workspace(dg.det_indexer_dk_workspace_size(128, 96, 128, 200, dg.IndexAddCfg(32)))
    assert_bitwise(run(inp, 32, ws=ws), want(inp, 32), "bad ids")
    assert dg.det_index_add_bad_ids(ws) == n_bad


def test_replay_under_load_and_atomic_arm(full):
    import torch
    w = want(full, 256)
    ids, p, t, q = dev_i32(full.ids), dev_f32(full.predict), dev_f32(full.target), dev_bf16(full.q)
    d0 = dev_f32(full.dk0)
    # the atomic arm starts from zero: its increments (about 1e-7 here) would be absorbed one by one
    # into an N(0, 1) start, which says nothing about the order of its adds
    zero = np.zeros_like(full.dk0)
    w0 = want(full, 256, dk0=zero)
    ws = dg.Workspace(dg.det_indexer_dk_workspace_size(4096, 512, 128, 8192))
    load = SideLoad()
    atoms = []
    for r in range(20):
        d = d0.clone()
        load.kick()
        dg.det_indexer_dk(d, ids, p, t, q, full.scale, cfg=dg.IndexAddCfg(256), ws=ws)
        assert_bitwise(host(d), w, "replay %d" % r)
        a = torch.zeros_like(d0)
        load.kick()
        dg.det_indexer_dk(a, ids, p, t, q, full.scale, atomic=True)
        atoms.append(host(a))
    load.wait()
    for a in atoms:
        assert rel_l2(a, w0) <= 1e-5
    distinct = len({a.tobytes() for a in atoms})
    note("indexer_dk atomic arm: %d distinct patterns in 20 runs" % distinct)
    assert distinct > 1, "the atomic arm is bit-stable here, so the replay check could not fail"
