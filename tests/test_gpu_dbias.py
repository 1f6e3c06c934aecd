"""GPU parity of det_grouped_dbias against the CPU oracle (bitwise), replay
stability under side-stream load, and the atomic arm's closeness."""
import numpy as np
import pytest

import deterministic_gradient_reductions_amd as dg
import workloads as W
from oracle import dbias as odb
from tests.gpu_util import SideLoad, assert_bitwise, dev_bf16, dev_f32, dev_i32, host, note, rel_l2

pytestmark = pytest.mark.gpu


def run(inp, offs=None, block_m=128, atomic=False, ld_pad=0, out_pad=0, stream=None, block_n=512):
    import torch
    M, N = inp.dA.shape
    if ld_pad:
        ab = np.zeros((M, N + ld_pad), np.uint16); ab[:, :N] = inp.dA
        dA = dev_bf16(ab)[:, :N]
    else:
        dA = dev_bf16(inp.dA)
    if out_pad:
        ob = np.zeros((inp.dbias0.shape[0], N + out_pad), np.float32); ob[:, :N] = inp.dbias0
        d = dev_f32(ob)[:, :N]
    else:
        d = dev_f32(inp.dbias0)
    o = dev_i32(inp.offs if offs is None else offs)
    torch.cuda.synchronize()
    cfg = None if block_n is None else dg.DbiasCfg(block_m, block_n)
    dg.det_grouped_dbias(d, dA, o, cfg=cfg, atomic=atomic, stream=stream)
    if stream is not None:
        stream.synchronize()
    return host(d)


@pytest.mark.parametrize("M,N,E,ld_pad", [(300, 2048, 4, 0), (1000, 520, 5, 0), (777, 64, 3, 8), (64, 8, 2, 0),
                                          (5, 16, 4, 0), (2500, 1032, 70, 16)])
@pytest.mark.parametrize("BM", [64, 128, 256])
def test_parity_small(M, N, E, ld_pad, BM):
    note("dbias parity M=%d N=%d E=%d ld_pad=%d block_m=%d" % (M, N, E, ld_pad, BM))
    inp = W.dbias_inputs(M=M, N=N, E=E, min_tokens=1, seed=41, out_init="normal")
    got = run(inp, block_m=BM, ld_pad=ld_pad, out_pad=4 if ld_pad else 0)
    assert_bitwise(got, odb.grouped_dbias(inp.dbias0, inp.dA, inp.offs, BM), "dbias")


@pytest.mark.parametrize("BN", [256, 128, None])
@pytest.mark.parametrize("M,N,E,ld_pad", [(1000, 520, 5, 0), (2500, 1032, 70, 16), (16384, 2048, 8, 0)])
def test_block_n_never_changes_bits(M, N, E, ld_pad, BN):
    """block_n (columns per workgroup) only shapes the launch: 256, 128 and the default (NULL)
    give the oracle's bits at block_m 128, including the full-size workload."""
    note("dbias block_n=%s M=%d N=%d E=%d" % (BN, M, N, E))
    inp = W.dbias_inputs(M=M, N=N, E=E, min_tokens=1, seed=43, out_init="normal")
    got = run(inp, block_m=128, ld_pad=ld_pad, out_pad=4 if ld_pad else 0, block_n=BN)
    assert_bitwise(got, odb.grouped_dbias(inp.dbias0, inp.dA, inp.offs, 128), "dbias block_n")


def test_offsets_clamped_and_empty_experts():
    inp = W.dbias_inputs(M=600, N=256, E=4, min_tokens=1, seed=42, out_init="normal")
    for offs in ([10, 10, 250, 130, 590], [0, 0, 0, 0, 0], [-7, 300, 300, 900, 900], [128, 256, 384, 512, 600]):
        offs = np.array(offs, np.int32)
        note("dbias offs %s" % offs.tolist())
        got = run(inp, offs=offs)
        assert_bitwise(got, odb.grouped_dbias(inp.dbias0, inp.dA, offs, 128), "dbias offs")


@pytest.mark.parametrize("BM", [128, 64, 256])
def test_full_size_parity_and_non_default_stream(BM):
    """Full size, every block_m: the last tile of the last expert ends at M, so
    a wave whose later row pieces lie past the tile must not read past M."""
    import torch
    inp = W.dbias_inputs(seed=6, out_init="normal")  # 16384 x 2048, E = 8
    note("dbias full size block_m=%d on a side stream" % BM)
    s = torch.cuda.Stream()
    got = run(inp, block_m=BM, stream=s)
    assert_bitwise(got, odb.grouped_dbias(inp.dbias0, inp.dA, inp.offs, BM), "dbias full")


def test_replay_under_load_and_atomic_arm():
    inp = W.dbias_inputs(M=8192, N=2048, E=8, min_tokens=64, seed=43, out_init="normal")
    ref = odb.grouped_dbias(inp.dbias0, inp.dA, inp.offs, 128)
    dA, o, d0 = dev_bf16(inp.dA), dev_i32(inp.offs), dev_f32(inp.dbias0)
    ws = dg.Workspace(dg.det_grouped_dbias_workspace_size(8192, 2048, 8))
    load = SideLoad()
    det, atom = [], []
    for i in range(20):
        d = d0.clone()
        load.kick()
        dg.det_grouped_dbias(d, dA, o, ws=ws)
        det.append(host(d).view(np.uint32).copy())
        a = d0.clone()
        load.kick()
        dg.det_grouped_dbias(a, dA, o, atomic=True)
        atom.append(host(a))
    load.wait()
    note("dbias replays done")
    for r in det:
        assert np.array_equal(r, ref.view(np.uint32))
    for a in atom:
        assert rel_l2(a - inp.dbias0, ref - inp.dbias0) <= 1e-5
    distinct = len({a.tobytes() for a in atom})
    note("dbias atomic arm: %d distinct bit patterns in 20 runs" % distinct)
    assert distinct > 1, "the atomic arm is bit-stable here, so the replay check could not fail"


def test_exact_integer_inputs_match_integer_sum():
    inp = W.dbias_inputs(M=5000, N=1024, E=6, min_tokens=1, seed=44, integer=True)
    x = inp.dA.astype(np.uint32) << 16
    xf = x.view(np.float32).astype(np.int64)
    exact = np.zeros(inp.dbias0.shape, np.int64)
    for e in range(6):
        exact[e] = xf[inp.offs[e]:inp.offs[e + 1]].sum(0)
    for atomic in (False, True):
        got = run(inp, atomic=atomic)
        assert np.array_equal(got.astype(np.int64), exact)
