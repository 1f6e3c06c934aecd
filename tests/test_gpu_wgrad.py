"""GPU checks of det_grouped_wgrad_acc (and its bf16 main_grad variant).

The oracle's split partial is the chain of the matrix-core step model
(oracle/mfma.py, checked against the instruction by test_gpu_mfma_model.py),
so the library's results are compared with the oracle bit for bit on general
inputs: every tile shape, split size and the full 8 x 1408 x 2048 workload on
the default kernel. Also:
  (i)   exact-integer inputs equal the exact integer sums, whole arrays, also at
        full size (any order gives them);
  (ii)  rel-L2 against the float64 definition <= 1e-5;
  (iii) the fold of the GPU's own split partials equals the full call;
  (iv)  bitwise replay under side-stream load; empty experts untouched;
  (v)   the atomic arm within rel-L2 1e-5, and with several splits per expert
        its bits vary from run to run (so the replay check can fail).
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

# output rows sampled at the full size: the edges of every 128-row wave band,
# the last m tile (its upper half has no rows) and random rows
FULL_ROWS = sorted(set([0, 1, 31, 32, 127, 128, 255, 256, 511, 512, 1023, 1024, 1151, 1152, 1279, 1280, 1281, 1406,
                        1407] + list(np.random.default_rng(99).choice(1408, 29, replace=False))))


def cfg(C, block_n=256, block_m=256):
    return dg.WgradCfg(block_m, block_n, 512, C)


def run(inp, C=0, atomic=False, mg0=None, offs=None, G=None, X=None, block_n=256, block_m=256, default=False):
    import torch
    Gd = dev_bf16(inp.G) if G is None else G
    Xd = dev_bf16(inp.X) if X is None else X
    mg = dev_f32(inp.main_grad0 if mg0 is None else mg0)
    o = dev_i32(inp.offs if offs is None else offs)
    torch.cuda.synchronize()
    dg.det_grouped_wgrad_acc(mg, Gd, Xd, o, cfg=None if default else cfg(C, block_n, block_m), atomic=atomic)
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


@pytest.mark.parametrize("bm,bn", TILES)
@pytest.mark.parametrize("C", [0, 1, 2, 4])
def test_bitwise_vs_oracle(C, bm, bn):
    """Realistic inputs, every tile and split size: bitwise the oracle (M = 384 leaves the 256-row tile a
    half-live last m tile; tails of 17 and 33 rows, an empty expert)."""
    inp = W.wgrad_inputs(E=5, M=384, N=1024, tokens=[1500, 0, 33, 2049, 17], seed=8, out_init="normal")
    note("wgrad bitwise C=%d tile %dx%d" % (C, bm, bn))
    got = run(inp, C, block_m=bm, block_n=bn)
    want = ow.grouped_wgrad_acc(inp.main_grad0, inp.G, inp.X, inp.offs, ktiles_per_split=C)
    assert_bitwise(got, want, "wgrad C=%d tile %dx%d" % (C, bm, bn))


@pytest.mark.parametrize("C", [0, 1, 4])
def test_fp64_rel_l2(C):
    inp = W.wgrad_inputs(E=3, M=M_, N=N_, tokens=[1024, 2600, 513], seed=4, out_init="zero")
    got = run(inp, C)
    ex = fp64.wgrad64(inp.main_grad0, inp.G, inp.X, inp.offs)
    err = rel_l2(got, ex)
    note("wgrad C=%d rel-L2 vs fp64 = %.3g" % (C, err))
    assert err <= 1e-5


def gpu_partial(inp, G, X, r0, r1, **kw):
    """Q for rows [r0, r1) as one split, computed by the GPU alone: -0.0 + Q = Q bitwise."""
    mg0 = np.full((1, inp.M, inp.N), -0.0, np.float32)
    return run(inp, 0, mg0=mg0, offs=np.array([r0, r1], np.int32), G=G, X=X, **kw)[0]


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
        for (a, b), q in zip(splits, parts):
            assert_bitwise(q, ow.chain_mfma(inp.G, inp.X, a, b), "split partial [%d, %d)" % (a, b))


@pytest.mark.parametrize("C", [0, 1])
def test_tile_shape_does_not_change_bits(C):
    inp = W.wgrad_inputs(E=5, M=384, N=1024, tokens=[1500, 0, 33, 2049, 640], seed=8, out_init="normal")
    G, X = dev_bf16(inp.G), dev_bf16(inp.X)
    outs = [run(inp, C, G=G, X=X, block_m=bm, block_n=bn) for bm, bn in TILES]
    note("wgrad C=%d: tiles %s" % (C, TILES))
    for (bm, bn), o in zip(TILES[1:], outs[1:]):
        assert_bitwise(o, outs[0], "tile %dx%d" % (bm, bn))


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
    inp = W.wgrad_inputs(E=4, M=M_, N=N_, tokens=[3000, 1024, 4100, 700], seed=7, out_init="normal")
    G, X, o = dev_bf16(inp.G), dev_bf16(inp.X), dev_i32(inp.offs)
    mg0 = dev_f32(inp.main_grad0)
    ex = fp64.wgrad64(inp.main_grad0, inp.G, inp.X, inp.offs)
    load = SideLoad()
    for C in (0, 2):
        ws = dg.Workspace(dg.det_grouped_wgrad_acc_workspace_size(int(inp.offs[-1]), 4, M_, N_, cfg(C)))
        pats = set()
        for r in range(20):
            mg = mg0.clone()
            load.kick()
            dg.det_grouped_wgrad_acc(mg, G, X, o, cfg=cfg(C), ws=ws)
            pats.add(host(mg).tobytes())
            a = mg0.clone()
            load.kick()
            dg.det_grouped_wgrad_acc(a, G, X, o, cfg=cfg(C), atomic=True)
            assert rel_l2(host(a) - inp.main_grad0, ex - inp.main_grad0) <= 1e-5
        load.wait()
        note("wgrad C=%d: det patterns %d (20 runs)" % (C, len(pats)))
        assert len(pats) == 1


# ------------------------------------------------------------------ full size
@pytest.fixture(scope="module")
def full():
    inp = W.wgrad_inputs(seed=5, out_init="normal")
    return inp, dev_bf16(inp.G), dev_bf16(inp.X)


@pytest.mark.parametrize("C", [0, 2])
def test_full_size_default_kernel_bitwise_vs_oracle(full, C):
    """E = 8, T_e ~ U{1024..8192}, 1408 x 2048 on the default 256 x 256 kernel (C = 0: the call with no
    configuration, as the benchmark makes it): sampled output rows of every expert, all columns, bitwise."""
    inp, G, X = full
    note("wgrad full size C=%d, T_total=%d, %d sampled rows" % (C, int(inp.offs[-1]), len(FULL_ROWS)))
    got = run(inp, C, G=G, X=X, default=(C == 0))
    want = ow.grouped_wgrad_acc(inp.main_grad0, inp.G, inp.X, inp.offs, ktiles_per_split=C, rows=FULL_ROWS)
    assert_bitwise(got[:, FULL_ROWS], want, "full size C=%d" % C)
    if C == 0:
        ex = fp64.wgrad64(inp.main_grad0, inp.G, inp.X, inp.offs)
        for e in range(8):
            err = rel_l2(got[e] - inp.main_grad0[e], ex[e] - inp.main_grad0[e])
            note("  expert %d (%d rows): rel-L2 vs fp64 %.3g" % (e, int(inp.offs[e + 1] - inp.offs[e]), err))
            assert err <= 1e-5


@pytest.mark.parametrize("C", [0, 2])
def test_full_size_exact_integers(C):
    inp = W.wgrad_inputs(seed=5, integer=True, out_init="normal")
    note("wgrad full size exact integers C=%d" % C)
    got = run(inp, C, default=(C == 0))
    assert np.array_equal(got.astype(np.float64), fp64.wgrad64(inp.main_grad0, inp.G, inp.X, inp.offs))


def test_full_size_fold_of_gpu_partials(full):
    """C = 2 at full size: the call equals the oracle's fold of the GPU's own split partials (expert 3)."""
    inp, G, X = full
    got = run(inp, 2, G=G, X=X)
    e = 3
    parts = [gpu_partial(inp, G, X, a, b) for a, b in ow.split_ranges(inp.offs, 512, 2)[e]]
    note("wgrad full size fold of %d GPU partials" % len(parts))
    assert_bitwise(got[e], ow.fold_partials(inp.main_grad0[e], parts), "fold")


def test_full_size_replay_under_load_and_varying_atomic_arm(full):
    """20 replays of the default call under side-stream load are bit-identical; the split-K atomic arm
    (C = 1: about 80 partials added into every element) gives more than one bit pattern."""
    import torch
    inp, G, X = full
    o = dev_i32(inp.offs)
    mg0 = dev_f32(inp.main_grad0)
    load = SideLoad()
    pats, apats = set(), set()
    mg = torch.empty_like(mg0)
    for r in range(20):
        mg.copy_(mg0)
        load.kick()
        dg.det_grouped_wgrad_acc(mg, G, X, o)
        pats.add(host(mg).tobytes())
        mg.copy_(mg0)
        load.kick()
        dg.det_grouped_wgrad_acc(mg, G, X, o, cfg=cfg(1), atomic=True)
        apats.add(host(mg).tobytes())
    load.wait()
    note("wgrad full size: det patterns %d, split-K atomic patterns %d (20 runs)" % (len(pats), len(apats)))
    assert len(pats) == 1
    assert len(apats) > 1


# ---------------------------------------------------------- bf16 main_grad
def run_bf16(inp, mg16, C=0, block_m=256, block_n=256, offs=None):
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
    inp = W.wgrad_inputs(E=4, M=M_, N=N_, tokens=[700, 0, 1300, 17], seed=3, integer=True)
    mg16 = bf16_init((4, M_, N_), 9, 4.0)
    note("wgrad bf16 exact integers C=%d" % C)
    got = run_bf16(inp, mg16, C)
    want = ow.grouped_wgrad_acc_bf16(mg16, inp.G, inp.X, inp.offs, ktiles_per_split=C)
    assert np.array_equal(got, want)
    assert np.array_equal(got[1], mg16[1])


@pytest.mark.parametrize("C,bm,bn", [(0, 128, 512), (2, 256, 256), (0, 256, 256), (1, 128, 256)])
def test_bf16_main_grad_bitwise_vs_oracle(C, bm, bn):
    inp = W.wgrad_inputs(E=3, M=M_, N=N_, tokens=[1500, 900, 0], seed=12)
    mg16 = bf16_init((3, M_, N_), 5, 0.01)
    note("wgrad bf16 vs oracle C=%d tile %dx%d" % (C, bm, bn))
    got = run_bf16(inp, mg16, C, block_m=bm, block_n=bn)
    assert np.array_equal(got, ow.grouped_wgrad_acc_bf16(mg16, inp.G, inp.X, inp.offs, ktiles_per_split=C))


def test_bf16_main_grad_full_size_replay(full):
    """The full workload (E = 8, 1408 x 2048, tiles 256 x 256, one split per expert): sampled rows bitwise
    against the oracle, and bitwise across two calls."""
    inp, _, _ = full
    mg16 = bf16_init((8, inp.M, inp.N), 6, 0.01)
    note("wgrad bf16 full size")
    a = run_bf16(inp, mg16, 0)
    b = run_bf16(inp, mg16, 0)
    assert np.array_equal(a, b)
    want = ow.grouped_wgrad_acc_bf16(mg16, inp.G, inp.X, inp.offs, rows=FULL_ROWS)
    assert np.array_equal(a[:, FULL_ROWS], want)
