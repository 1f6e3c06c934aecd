"""GPU checks of det_grouped_wgrad_acc.

The pages say nothing about how a matrix-core instruction rounds inside one
multiply-accumulate, so the oracle cannot reproduce a split's MFMA chain bit
for bit ("parity unpinned" for the chain). What is pinned here:
  (i)   exact-integer inputs: every partial sum is an exactly representable
        integer, so any order gives the exact integer result, bit for bit;
  (ii)  realistic inputs: rel-L2 against the float64 definition <= 1e-5;
  (iii) the split structure, the ordered fold and the main_grad add: each
        split's partial Q_s is obtained from the GPU alone (a one-expert call on
        exactly that split's rows into a -0.0 slice returns Q_s bitwise), and the
        oracle's fold RN32(main_grad + ((Q_0 + Q_1) + ...)) must equal the full
        call bit for bit;
  (iv)  bitwise replay under side-stream load; empty experts untouched;
  (v)   the atomic arm within rel-L2 1e-5.
"""
import numpy as np
import pytest

import deterministic_gradient_reductions_amd as dg
import workloads as W
from oracle import fp64, wgrad as ow
from tests.gpu_util import SideLoad, assert_bitwise, dev_bf16, dev_f32, dev_i32, host, note, rel_l2

pytestmark = pytest.mark.gpu

M_, N_ = 256, 512  # small shapes: 2 x 2 workgroup tiles


TILES = [(128, 256), (128, 512), (256, 256)]


def cfg(C, block_n=512, block_m=128):
    return dg.WgradCfg(block_m, block_n, 512, C)


def run(inp, C=0, atomic=False, mg0=None, offs=None, G=None, X=None, block_n=512, block_m=128):
    import torch
    Gd = dev_bf16(inp.G) if G is None else G
    Xd = dev_bf16(inp.X) if X is None else X
    mg = dev_f32(inp.main_grad0 if mg0 is None else mg0)
    o = dev_i32(inp.offs if offs is None else offs)
    torch.cuda.synchronize()
    dg.det_grouped_wgrad_acc(mg, Gd, Xd, o, cfg=cfg(C, block_n, block_m), atomic=atomic)
    return host(mg)


@pytest.mark.parametrize("C", [0, 1, 2])
def test_exact_integer_inputs(C):
    inp = W.wgrad_inputs(E=4, M=M_, N=N_, tokens=[700, 0, 1300, 17], seed=3, integer=True, out_init="normal")
    note("wgrad exact integers C=%d" % C)
    got = run(inp, C)
    exact = fp64.wgrad64(inp.main_grad0, inp.G, inp.X, inp.offs)
    assert np.array_equal(got.astype(np.float64), exact)
    assert_bitwise(got[1], inp.main_grad0[1], "empty expert")
    got_a = run(inp, C, atomic=True)
    assert np.array_equal(got_a.astype(np.float64), exact)


@pytest.mark.parametrize("C", [0, 1, 4])
def test_fp64_rel_l2(C):
    inp = W.wgrad_inputs(E=3, M=M_, N=N_, tokens=[1024, 2600, 513], seed=4, out_init="zero")
    got = run(inp, C)
    ex = fp64.wgrad64(inp.main_grad0, inp.G, inp.X, inp.offs)
    err = rel_l2(got, ex)
    note("wgrad C=%d rel-L2 vs fp64 = %.3g" % (C, err))
    assert err <= 1e-5


def gpu_partial(inp, G, X, r0, r1):
    """Q for rows [r0, r1) as one split, computed by the GPU alone: -0.0 + Q = Q bitwise."""
    mg0 = np.full((1, inp.M, inp.N), -0.0, np.float32)
    return run(inp, 0, mg0=mg0, offs=np.array([r0, r1], np.int32), G=G, X=X)[0]


@pytest.mark.parametrize("C", [1, 2])
def test_fold_of_gpu_partials_matches_oracle(C):
    inp = W.wgrad_inputs(E=3, M=M_, N=N_, tokens=[1500, 512, 2049], seed=5, out_init="normal")
    G, X = dev_bf16(inp.G), dev_bf16(inp.X)
    full = run(inp, C, G=G, X=X)
    for e, splits in enumerate(ow.split_ranges(inp.offs, 512, C)):
        parts = [gpu_partial(inp, G, X, a, b) for a, b in splits]
        want = ow.fold_partials(inp.main_grad0[e], parts)
        note("wgrad C=%d expert %d: %d splits" % (C, e, len(parts)))
        assert_bitwise(full[e], want, "fold expert %d" % e)
    # one split per expert: the epilogue adds the partial directly
    single = run(inp, 0, G=G, X=X)
    for e in range(3):
        a, b = int(inp.offs[e]), int(inp.offs[e + 1])
        assert_bitwise(single[e], ow.fold_partials(inp.main_grad0[e], [gpu_partial(inp, G, X, a, b)]), "single")


@pytest.mark.parametrize("C", [0, 1])
def test_tile_shape_does_not_change_bits(C):
    """128x256, 128x512 and 256x256 workgroup tiles give the same bits (the tile only shapes the launch).

    M = 384 leaves the 256-row tile a 128-row tail, whose second half of waves has no rows.
    """
    inp = W.wgrad_inputs(E=5, M=384, N=1024, tokens=[1500, 0, 33, 2049, 640], seed=8, out_init="normal")
    G, X = dev_bf16(inp.G), dev_bf16(inp.X)
    outs = [run(inp, C, G=G, X=X, block_m=bm, block_n=bn) for bm, bn in TILES]
    note("wgrad C=%d: tiles %s" % (C, TILES))
    for (bm, bn), o in zip(TILES[1:], outs[1:]):
        assert_bitwise(o, outs[0], "tile %dx%d" % (bm, bn))
    ex = fp64.wgrad64(inp.main_grad0, inp.G, inp.X, inp.offs)
    assert rel_l2(outs[0] - inp.main_grad0, ex - inp.main_grad0) <= 1e-5


@pytest.mark.parametrize("bm,bn", TILES)
def test_exact_integer_inputs_every_tile(bm, bn):
    inp = W.wgrad_inputs(E=4, M=384, N=512, tokens=[700, 0, 1300, 17], seed=9, integer=True, out_init="normal")
    note("wgrad exact integers tile %dx%d" % (bm, bn))
    got = run(inp, 0, block_m=bm, block_n=bn)
    assert np.array_equal(got.astype(np.float64), fp64.wgrad64(inp.main_grad0, inp.G, inp.X, inp.offs))
    assert_bitwise(got[1], inp.main_grad0[1], "empty expert")


def test_partial_is_independent_of_position():
    """A split's bits depend only on its rows: the same rows at another offset give the same partial."""
    inp = W.wgrad_inputs(E=1, M=M_, N=N_, tokens=[2000], seed=6)
    G, X = dev_bf16(inp.G), dev_bf16(inp.X)
    q1 = gpu_partial(inp, G, X, 100, 900)
    shifted = W.WgradInputs(M_, N_, inp.offs, np.roll(inp.G, 37, axis=0), np.roll(inp.X, 37, axis=0),
                            inp.main_grad0)
    q2 = gpu_partial(shifted, dev_bf16(shifted.G), dev_bf16(shifted.X), 137, 937)
    assert_bitwise(q1, q2, "position")


def test_replay_under_load_and_atomic_arm():
    import torch
    inp = W.wgrad_inputs(E=4, M=M_, N=N_, tokens=[3000, 1024, 4100, 700], seed=7, out_init="normal")
    G, X, o = dev_bf16(inp.G), dev_bf16(inp.X), dev_i32(inp.offs)
    mg0 = dev_f32(inp.main_grad0)
    ex = fp64.wgrad64(inp.main_grad0, inp.G, inp.X, inp.offs)
    load = SideLoad()
    for C in (0, 2):
        ws = dg.Workspace(dg.det_grouped_wgrad_acc_workspace_size(int(inp.offs[-1]), 4, M_, N_, cfg(C)))
        pats, apats = set(), set()
        for r in range(20):
            mg = mg0.clone()
            load.kick()
            dg.det_grouped_wgrad_acc(mg, G, X, o, cfg=cfg(C), ws=ws)
            pats.add(host(mg).tobytes())
            a = mg0.clone()
            load.kick()
            dg.det_grouped_wgrad_acc(a, G, X, o, cfg=cfg(C), atomic=True)
            ah = host(a)
            apats.add(ah.tobytes())
            assert rel_l2(ah - inp.main_grad0, ex - inp.main_grad0) <= 1e-5
        load.wait()
        note("wgrad C=%d: det patterns %d, atomic patterns %d (20 runs)" % (C, len(pats), len(apats)))
        assert len(pats) == 1


def test_full_size_sampled():
    """Full workload (E=8, T_e ~ U{1024..8192}, 1408 x 2048): rel-L2 vs fp64 on sampled experts and rows."""
    inp = W.wgrad_inputs(seed=5, out_init="normal")
    note("wgrad full size T_total=%d" % int(inp.offs[-1]))
    got = run(inp, 0)
    for e in (0, 3, 7):
        a, b = int(inp.offs[e]), int(inp.offs[e + 1])
        rows = np.random.default_rng(e).choice(1408, 64, replace=False)
        Gf = fp64.widen(inp.G[a:b]); Xf = fp64.widen(inp.X[a:b])
        ex = inp.main_grad0[e][rows].astype(np.float64) + Gf[:, rows].T @ Xf
        assert rel_l2(got[e][rows] - inp.main_grad0[e][rows], ex - inp.main_grad0[e][rows]) <= 1e-5


def run_bf16(inp, mg16, C=0, block_m=128, block_n=512, offs=None):
    """det_grouped_wgrad_acc_bf16 on bf16 main_grad bits; returns the bits after the call."""
    import torch
    Gd, Xd = dev_bf16(inp.G), dev_bf16(inp.X)
    mg = torch.from_numpy(np.ascontiguousarray(mg16).view(np.int16)).cuda().view(torch.bfloat16)
    o = dev_i32(inp.offs if offs is None else offs)
    torch.cuda.synchronize()
    dg.det_grouped_wgrad_acc_bf16(mg, Gd, Xd, o, cfg=cfg(C, block_n, block_m))
    return mg.view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_init(shape, seed, scale=1.0):
    from oracle.primitives import narrow_bf16
    return narrow_bf16((np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32))


@pytest.mark.parametrize("C", [0, 1, 3])
def test_bf16_main_grad_exact_integers(C):
    """Integer inputs: bitwise the oracle's bf16 accumulate of the exact dW; the
    empty expert keeps its bits."""
    inp = W.wgrad_inputs(E=4, M=M_, N=N_, tokens=[700, 0, 1300, 17], seed=3, integer=True)
    mg16 = bf16_init((4, M_, N_), 9, 4.0)
    note("wgrad bf16 exact integers C=%d" % C)
    got = run_bf16(inp, mg16, C)
    want = ow.grouped_wgrad_acc_bf16(mg16, inp.G, inp.X, inp.offs, ktiles_per_split=C)
    assert np.array_equal(got, want)
    assert np.array_equal(got[1], mg16[1])


@pytest.mark.parametrize("C,bm,bn", [(0, 128, 512), (2, 256, 256), (0, 256, 256)])
def test_bf16_main_grad_is_bf16_add_of_the_fp32_dw(C, bm, bn):
    """Realistic inputs: the bf16 result equals the oracle's bf16 accumulate of
    the float32 dW that det_grouped_wgrad_acc produces with the same tiles and
    splits (into a -0.0 main_grad, which returns dW itself), bit for bit."""
    inp = W.wgrad_inputs(E=3, M=M_, N=N_, tokens=[1500, 900, 0], seed=12)
    note("wgrad bf16 vs fp32 dW C=%d tile %dx%d" % (C, bm, bn))
    dW = run(inp, C=C, mg0=np.full((3, M_, N_), -0.0, np.float32), block_m=bm, block_n=bn)
    mg16 = bf16_init((3, M_, N_), 5, 0.01)
    got = run_bf16(inp, mg16, C, block_m=bm, block_n=bn)
    want = mg16.copy()
    for e in range(2):
        want[e] = ow.accumulate_bf16(mg16[e], dW[e])
    assert np.array_equal(got, want)


def test_bf16_main_grad_full_size_replay():
    """The scale workload (E = 8, 1408 x 2048, tiles 256 x 256, one split per
    expert): bitwise against the oracle's bf16 add of the fp32 path's dW, and
    bitwise across two calls."""
    inp = W.wgrad_inputs(seed=5)
    E, M, N = 8, inp.M, inp.N
    note("wgrad bf16 full size")
    dW = run(inp, C=0, mg0=np.full((E, M, N), -0.0, np.float32), block_m=256, block_n=256)
    mg16 = bf16_init((E, M, N), 6, 0.01)
    a = run_bf16(inp, mg16, 0, block_m=256, block_n=256)
    b = run_bf16(inp, mg16, 0, block_m=256, block_n=256)
    assert np.array_equal(a, b)
    for e in range(E):
        assert np.array_equal(a[e], ow.accumulate_bf16(mg16[e], dW[e])), e
