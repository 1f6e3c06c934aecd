"""GPU parity of det_grouped_dprob against the CPU oracle (bitwise), replay
stability under side-stream load, and the atomic arm's closeness."""
import numpy as np
import pytest

import deterministic_gradient_reductions_amd as dg
import workloads as W
from oracle import dprob as od
from tests.gpu_util import SideLoad, assert_bitwise, dev_bf16, dev_f32, dev_i32, host, note, rel_l2

pytestmark = pytest.mark.gpu


def run(inp, offs=None, cfg=None, atomic=False, ld_pad=0, stream=None):
    import torch
    M, N = inp.dY.shape
    if ld_pad:
        yb = np.zeros((M, N + ld_pad), np.uint16); yb[:, :N] = inp.dY
        cb = np.zeros((M, N + ld_pad), np.uint16); cb[:, :N] = inp.C
        dY = dev_bf16(yb)[:, :N]; C = dev_bf16(cb)[:, :N]
    else:
        dY = dev_bf16(inp.dY); C = dev_bf16(inp.C)
    d = dev_f32(inp.dprob0)
    o = dev_i32(inp.offs if offs is None else offs)
    torch.cuda.synchronize()
    dg.det_grouped_dprob(d, dY, C, o, cfg=cfg, atomic=atomic, stream=stream)
    if stream is not None:
        stream.synchronize()
    return host(d)


@pytest.mark.parametrize("M,N,ld_pad", [(300, 2048, 0), (77, 300, 0), (64, 1000, 0), (33, 2056, 8), (50, 130, 3),
                                        (5, 1, 0), (1, 4096, 0)])
def test_parity_small(M, N, ld_pad):
    note("dprob parity M=%d N=%d ld_pad=%d" % (M, N, ld_pad))
    inp = W.dprob_inputs(M=M, N=N, E=4, min_tokens=1, seed=21, out_init="normal")
    got = run(inp, ld_pad=ld_pad)
    assert_bitwise(got, od.grouped_dprob(inp.dprob0, inp.dY, inp.C, inp.offs), "dprob")


def test_offs_range_and_empty_experts():
    inp = W.dprob_inputs(M=200, N=512, E=3, min_tokens=1, seed=22, out_init="normal")
    for offs in ([10, 10, 50, 150], [0, 0, 0, 0], [190, 195, 300, 300], [-5, 7, 9, 20]):
        offs = np.array(offs, np.int32)
        note("dprob offs %s" % offs.tolist())
        got = run(inp, offs=offs)
        assert_bitwise(got, od.grouped_dprob(inp.dprob0, inp.dY, inp.C, offs), "dprob offs")


def test_rows_per_wg_does_not_change_bits():
    inp = W.dprob_inputs(M=1000, N=2048, E=8, min_tokens=8, seed=23, out_init="normal")
    ref = od.grouped_dprob(inp.dprob0, inp.dY, inp.C, inp.offs)
    for r in (1, 3, 16, 64, 1024):
        note("dprob rows_per_wg=%d" % r)
        assert_bitwise(run(inp, cfg=dg.DprobCfg(128, r)), ref, "rows_per_wg")


def test_full_size_parity_and_non_default_stream():
    import torch
    inp = W.dprob_inputs(seed=4, out_init="normal")  # 16384 x 2048, E=8
    note("dprob full size on a side stream")
    s = torch.cuda.Stream()
    got = run(inp, stream=s)
    assert_bitwise(got, od.grouped_dprob(inp.dprob0, inp.dY, inp.C, inp.offs), "dprob full")


def test_replay_under_load_and_atomic_arm():
    import torch
    inp = W.dprob_inputs(M=16384, N=2048, E=8, min_tokens=64, seed=24, out_init="normal")
    ref = od.grouped_dprob(inp.dprob0, inp.dY, inp.C, inp.offs)
    dY, C, o = dev_bf16(inp.dY), dev_bf16(inp.C), dev_i32(inp.offs)
    d0 = dev_f32(inp.dprob0)
    load = SideLoad()
    det, atom = [], []
    for i in range(20):
        d = d0.clone()
        load.kick()
        dg.det_grouped_dprob(d, dY, C, o)
        det.append(host(d).view(np.uint32).copy())
        a = d0.clone()
        load.kick()
        dg.det_grouped_dprob(a, dY, C, o, atomic=True)
        atom.append(host(a))
    load.wait()
    note("dprob replays done")
    for r in det:
        assert np.array_equal(r, ref.view(np.uint32))
    for a in atom:
        assert rel_l2(a - inp.dprob0, ref - inp.dprob0) <= 1e-5
    distinct = len({a.tobytes() for a in atom})
    note("dprob atomic arm: %d distinct bit patterns in 20 runs" % distinct)
    assert distinct > 1, "the atomic arm is bit-stable here, so the replay check could not fail"


def test_exact_integer_inputs_match_integer_sum():
    rng = np.random.default_rng(5)
    M, N = 256, 2048
    dYf = rng.integers(-4, 5, (M, N)).astype(np.float32); Cf = rng.integers(-4, 5, (M, N)).astype(np.float32)
    inp = W.DprobInputs(M, N, np.array([0, 100, 256], np.int32), W.bf16_bits(dYf), W.bf16_bits(Cf),
                        np.zeros(M, np.float32))
    got = run(inp)
    exact = (dYf.astype(np.int64) * np.maximum(Cf, 0).astype(np.int64) ** 2).sum(1)
    assert np.array_equal(got.astype(np.int64), exact)
    got_a = run(inp, atomic=True)
    assert np.array_equal(got_a.astype(np.int64), exact)
