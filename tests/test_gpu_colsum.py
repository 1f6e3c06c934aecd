"""GPU parity of det_colsum and of the device detmath against the CPU oracle
(bitwise), tile-config coverage, strided views, replay under load and the
atomic arm's closeness."""
import numpy as np
import pytest

import deterministic_gradient_reductions_amd as dg
import workloads as W
from oracle import colsum as oc, detmath as dm
from tests.gpu_util import SideLoad, assert_bitwise, dev_bf16, dev_f32, host, note, rel_l2

pytestmark = pytest.mark.gpu


def detmath_sample():
    rng = np.random.default_rng(99)
    parts = [rng.uniform(-110, 95, 4_000_000), rng.uniform(-25, 25, 4_000_000), rng.uniform(-1, 1, 2_000_000),
             np.exp2(rng.uniform(-149, 127, 2_000_000)) * rng.choice([-1, 1], 2_000_000),
             np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 20.0, 20.000002, 89.0, 89.00001, -104.0, -104.00001,
                       88.72283, -87.33655, 1e-45, -1e-45, 1.17549435e-38])]
    x = np.concatenate(parts).astype(np.float32)
    # every float32 whose upper 16 bits are a bf16 value (the gate's x = a + dt_bias covers these densely)
    allbf = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    return np.concatenate([x, allbf, allbf + np.float32(0.37)])


@pytest.mark.parametrize("fn", ["exp32", "log1p32", "softplus32", "sigmoid32"])
def test_detmath_bitwise(fn):
    import torch
    x = detmath_sample()
    if fn == "log1p32":
        x = np.abs(x[np.isfinite(x)]).astype(np.float32)
        x = np.concatenate([x[x <= 1.0], np.random.default_rng(1).uniform(0, 1, 4_000_000).astype(np.float32)])
    note("detmath %s on %d inputs" % (fn, x.size))
    xd = dev_f32(x); yd = torch.empty_like(xd)
    dg.det_detmath_eval(xd, yd, fn)
    got = host(yd)
    with np.errstate(all="ignore"):
        want = getattr(dm, fn)(x)
    g, w = got.view(np.uint32), want.view(np.uint32)
    both_nan = np.isnan(got) & np.isnan(want)
    bad = np.nonzero((g != w) & ~both_nan)[0]
    assert len(bad) == 0, "%d mismatches, first x=%r gpu=%r cpu=%r" % (len(bad), x[bad[0]], got[bad[0]], want[bad[0]])


def run(inp, cfg=None, atomic=False, transpose=False, dA0=None, ddt0=None, ws=None):
    import torch
    T, H = inp.a.shape
    dev_in = dev_f32 if inp.a.dtype == np.float32 else dev_bf16  # float32 values or bf16 bits
    a = dev_in(inp.a)
    dgb = dev_in(inp.dg_base)
    d = dgb[:, H:]  # strided view: row stride 2H, offset H
    if transpose:
        a = dev_in(np.ascontiguousarray(inp.a.T)).t()
        d = dev_in(np.ascontiguousarray(inp.dg.T)).t()
    o1 = dev_f32(inp.dA_log0 if dA0 is None else dA0)
    o2 = dev_f32(inp.ddt_bias0 if ddt0 is None else ddt0)
    torch.cuda.synchronize()
    dg.det_colsum(a, d, dev_f32(inp.A_log), dev_f32(inp.dt_bias), o1, o2, cfg=cfg, atomic=atomic, ws=ws)
    return host(o1), host(o2)


def oracle(inp, bt, dA0=None, ddt0=None):
    return oc.colsum(inp.a, inp.dg, inp.A_log, inp.dt_bias, inp.dA_log0 if dA0 is None else dA0,
                     inp.ddt_bias0 if ddt0 is None else ddt0, bt)


@pytest.mark.parametrize("bt", [64, 128, 256])
@pytest.mark.parametrize("bh", [8, 16, 32])
def test_train_shape_all_cfgs_with_tail(bt, bh):
    for T in (16384, 16323):
        inp = W.gate_inputs(T, 32, seed=2, out_init="normal")
        note("colsum T=%d H=32 cfg=%dx%d" % (T, bt, bh))
        r1, r2 = run(inp, cfg=dg.ColsumCfg(bt, bh))
        w1, w2 = oracle(inp, bt)
        assert_bitwise(r1, w1, "dA_log"); assert_bitwise(r2, w2, "ddt_bias")


def test_tiny_shape_default_cfg_and_selector():
    inp = W.gate_inputs(4096, 16, seed=1, out_init="zero")
    c = dg.det_colsum_select_cfg(4096, 16)
    r1, r2 = run(inp)
    w1, w2 = oracle(inp, c.block_t)
    assert_bitwise(r1, w1, "dA_log"); assert_bitwise(r2, w2, "ddt_bias")


# (700, 300): 38 head groups of 8 over tile groups of 8 with a short last group;
# (300000, 3): a fold of several full 1024-tile rounds and a partial one at block_t 64
@pytest.mark.parametrize("T,H", [(1, 1), (63, 5), (1000, 40), (2049, 3), (300, 33), (33000, 2), (70001, 3),
                                 (700, 300), (300000, 3)])
def test_ragged_heads_and_rows(T, H):
    inp = W.gate_inputs(T, H, seed=7, out_init="normal")
    for bt, bh in ((64, 8), (256, 32), (128, 16)):
        note("colsum ragged T=%d H=%d cfg=%dx%d" % (T, H, bt, bh))
        r1, r2 = run(inp, cfg=dg.ColsumCfg(bt, bh))
        w1, w2 = oracle(inp, bt)
        assert_bitwise(r1, w1, "dA_log"); assert_bitwise(r2, w2, "ddt_bias")


def test_transposed_views():
    inp = W.gate_inputs(777, 12, seed=8, out_init="normal")
    r1, r2 = run(inp, cfg=dg.ColsumCfg(128, 16), transpose=True)
    w1, w2 = oracle(inp, 128)
    assert_bitwise(r1, w1, "dA_log"); assert_bitwise(r2, w2, "ddt_bias")


def test_microbatch_accumulation_and_ticket_reuse():
    """Four accumulated microbatches through one workspace equal the oracle applied four times."""
    inp = W.gate_inputs(4 * 4096, 32, seed=9, out_init="normal")
    ws = dg.Workspace(dg.det_colsum_workspace_size(4096, 32, dg.ColsumCfg(128, 32)))
    o1, o2 = inp.dA_log0, inp.ddt_bias0
    w1, w2 = inp.dA_log0, inp.ddt_bias0
    for mb in range(4):
        sl = slice(mb * 4096, (mb + 1) * 4096)
        part = W.GateInputs(4096, 32, inp.a[sl], inp.dg_base[sl], inp.A_log, inp.dt_bias, o1, o2)
        o1, o2 = run(part, cfg=dg.ColsumCfg(128, 32), ws=ws)
        w1, w2 = oc.colsum(inp.a[sl], inp.dg[sl], inp.A_log, inp.dt_bias, w1, w2, 128)
    assert_bitwise(o1, w1, "dA_log"); assert_bitwise(o2, w2, "ddt_bias")


def test_replay_under_load_and_atomic_arm():
    import torch
    inp = W.gate_inputs(16384, 32, seed=2, out_init="normal")
    cfg = dg.ColsumCfg(128, 32)
    w1, w2 = oracle(inp, 128)
    a = dev_bf16(inp.a); d = dev_bf16(inp.dg_base)[:, 32:]
    Al, db = dev_f32(inp.A_log), dev_f32(inp.dt_bias)
    load = SideLoad()
    atoms = []
    for i in range(20):
        o1, o2 = dev_f32(inp.dA_log0), dev_f32(inp.ddt_bias0)
        load.kick()
        dg.det_colsum(a, d, Al, db, o1, o2, cfg=cfg)
        assert_bitwise(host(o1), w1, "replay dA_log"); assert_bitwise(host(o2), w2, "replay ddt_bias")
        p1, p2 = dev_f32(inp.dA_log0), dev_f32(inp.ddt_bias0)
        load.kick()
        dg.det_colsum(a, d, Al, db, p1, p2, cfg=cfg, atomic=True)
        atoms.append((host(p1), host(p2)))
    load.wait()
    for p1, p2 in atoms:
        assert rel_l2(p1 - inp.dA_log0, w1 - inp.dA_log0) <= 1e-5
        assert rel_l2(p2 - inp.ddt_bias0, w2 - inp.ddt_bias0) <= 1e-5
    distinct = len({(x.tobytes(), y.tobytes()) for x, y in atoms})
    note("colsum atomic arm: %d distinct patterns in 20 runs" % distinct)
    assert distinct > 1, "the atomic arm is bit-stable here, so the replay check could not fail"


def test_block_h_never_changes_bits():
    inp = W.gate_inputs(5000, 24, seed=10, out_init="normal")
    base = run(inp, cfg=dg.ColsumCfg(128, 8))
    for bh in (16, 32):
        r = run(inp, cfg=dg.ColsumCfg(128, bh))
        assert_bitwise(r[0], base[0], "bh"); assert_bitwise(r[1], base[1], "bh")


@pytest.mark.parametrize("T,H,bt", [(16384, 32, 64), (16323, 32, 128), (1000, 40, 256), (70001, 3, 64)])
def test_f32_inputs(T, H, bt):
    """float32 a and dg (strided dg view, tails, multi-round folds): bitwise against the oracle."""
    inp = W.gate_inputs(T, H, seed=12, out_init="normal", dtype="f32")
    note("colsum f32 inputs T=%d H=%d block_t=%d" % (T, H, bt))
    r1, r2 = run(inp, cfg=dg.ColsumCfg(bt, 8))
    w1, w2 = oracle(inp, bt)
    assert_bitwise(r1, w1, "dA_log f32"); assert_bitwise(r2, w2, "ddt_bias f32")


def test_f32_inputs_transposed_and_atomic_arm():
    inp = W.gate_inputs(777, 12, seed=13, out_init="normal", dtype="f32")
    r1, r2 = run(inp, cfg=dg.ColsumCfg(128, 16), transpose=True)
    w1, w2 = oracle(inp, 128)
    assert_bitwise(r1, w1, "dA_log f32 T"); assert_bitwise(r2, w2, "ddt_bias f32 T")
    a1, a2 = run(inp, cfg=dg.ColsumCfg(128, 16), atomic=True)
    assert rel_l2(a1 - inp.dA_log0, w1 - inp.dA_log0) <= 1e-5 and rel_l2(a2 - inp.ddt_bias0, w2 - inp.ddt_bias0) <= 1e-5


def run_da(inp, cfg=None, atomic=False, da_layout="rows"):
    """det_colsum_da: returns (dA_log, ddt_bias, da) with da as stored (bf16 bits or float32)."""
    import torch
    T, H = inp.a.shape
    f32 = inp.a.dtype == np.float32
    dev_in = dev_f32 if f32 else dev_bf16
    a = dev_in(inp.a)
    d = dev_in(inp.dg_base)[:, H:]
    o1, o2 = dev_f32(inp.dA_log0), dev_f32(inp.ddt_bias0)
    dt = torch.float32 if f32 else torch.bfloat16
    if da_layout == "rows":
        da = torch.full((T, H), float("nan"), dtype=dt, device="cuda")
    elif da_layout == "cols":  # column-major: a transposed view
        da = torch.full((H, T), float("nan"), dtype=dt, device="cuda").t()
    else:  # a column slice of a wider tensor
        da = torch.full((T, 3 * H), float("nan"), dtype=dt, device="cuda")[:, H:2 * H]
    torch.cuda.synchronize()
    dg.det_colsum_da(a, d, dev_f32(inp.A_log), dev_f32(inp.dt_bias), o1, o2, da, cfg=cfg, atomic=atomic)
    out = da.contiguous().cpu()
    out = out.numpy() if f32 else out.view(torch.int16).numpy().view(np.uint16)
    return host(o1), host(o2), out


@pytest.mark.parametrize("dtype,T,H,layout", [("bf16", 16384, 32, "rows"), ("bf16", 1000, 12, "cols"),
                                              ("f32", 4096, 16, "slice"), ("f32", 333, 5, "rows")])
def test_da_output(dtype, T, H, layout):
    """da bitwise against the oracle (bf16 round to nearest even, or float32),
    and dA_log / ddt_bias bitwise those of det_colsum, on both arms."""
    note("colsum_da %s T=%d H=%d %s" % (dtype, T, H, layout))
    inp = W.gate_inputs(T=T, H=H, seed=T + H, out_init="normal", dtype=dtype)
    want_da = oc.gate_da(inp.a, inp.dg, inp.A_log, inp.dt_bias)
    c = dg.det_colsum_select_cfg(T, H)
    w1, w2 = oc.colsum(inp.a, inp.dg, inp.A_log, inp.dt_bias, inp.dA_log0, inp.ddt_bias0, c.block_t)
    g1, g2, gda = run_da(inp, da_layout=layout)
    assert np.array_equal(gda.view(np.uint16 if dtype == "bf16" else np.uint32),
                          want_da.view(np.uint16 if dtype == "bf16" else np.uint32)), "da"
    assert_bitwise(g1, w1, "dA_log"); assert_bitwise(g2, w2, "ddt_bias")
    a1, a2, ada = run_da(inp, atomic=True, da_layout=layout)
    assert np.array_equal(ada.view(np.uint8), gda.view(np.uint8)), "da on the atomic arm"
    assert rel_l2(a1, w1) < 1e-5 and rel_l2(a2, w2) < 1e-5
