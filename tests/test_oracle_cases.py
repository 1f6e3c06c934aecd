"""Pins of the four oracle cases (CPU): fp64 bounds, exact integers, order probes,
brute force and invariants. None of these compares the oracle with itself."""
import numpy as np
import pytest

import workloads as W
from oracle import brute, colsum as oc, dbias as odb, dprob as od, fp64, index_add as oi, wgrad as ow
from oracle.primitives import narrow_bf16, widen_bf16

U = 2.0 ** -24


def gamma(d):
    return d * U / (1 - d * U)


def rel_l2(a, b):
    a = np.asarray(a, np.float64); b = np.asarray(b, np.float64)
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


def bits(x):
    return np.asarray(x, np.float32).view(np.uint32)


# ----------------------------------------------------------------------- dprob
@pytest.mark.parametrize("M,N", [(64, 2048), (37, 300), (5, 128), (3, 1)])
def test_dprob_fp64_bound(M, N):
    inp = W.dprob_inputs(M=M, N=N, E=4, min_tokens=1, seed=7, out_init="normal")
    got = od.grouped_dprob(inp.dprob0, inp.dY, inp.C, inp.offs)
    exact, absum = fp64.dprob64(inp.dprob0, inp.dY, inp.C, inp.offs)
    n_tiles = -(-N // 128)
    d = 7 + n_tiles + 1  # tree depth + fold length + final add
    bound = gamma(d) * (absum + np.abs(inp.dprob0)) + 2.0 ** -149
    assert np.all(np.abs(got - exact) <= bound)
    assert rel_l2(got, exact) <= 1e-5


def test_dprob_exact_integers():
    rng = np.random.default_rng(3)
    M, N = 16, 2048
    dY = W.bf16_bits(rng.integers(-4, 5, (M, N)).astype(np.float32))
    C = W.bf16_bits(rng.integers(-4, 5, (M, N)).astype(np.float32))
    d0 = rng.integers(-100, 100, M).astype(np.float32)
    offs = np.array([0, 5, 16], np.int32)
    got = od.grouped_dprob(d0, dY, C, offs)
    y = widen_bf16(dY).astype(np.int64); c = widen_bf16(C).astype(np.int64)
    exact = d0.astype(np.int64) + (y * np.maximum(c, 0) ** 2).sum(1)
    assert np.array_equal(got.astype(np.int64), exact)


def test_dprob_order_probe():
    """+-M inside one tile and across tiles reveals tree-then-fold order."""
    M_ = 2.0 ** 40
    rows = []
    cases = [(0, 1), (0, 127), (5, 70), (128, 129), (100, 300), (0, 2047), (1500, 1600)]
    N = 2048
    for p, q in cases:
        y = np.ones(N, np.float32); y[p], y[q] = M_, -M_
        rows.append(y)
    dY = W.bf16_bits(np.stack(rows)); C = W.bf16_bits(np.ones((len(rows), N), np.float32))
    got = od.grouped_dprob(np.zeros(len(rows), np.float32), dY, C, np.array([0, len(rows)], np.int32))
    for r, (p, q) in enumerate(cases):
        tp, tq = p // 128, q // 128
        if tp == tq:
            # within a tile: tree value n - 2^bitlen(p^q); other tiles add 128 each after it
            exp_val = (128 - 2 ** int((p % 128) ^ (q % 128)).bit_length()) + 128 * (N // 128 - 1)
        else:
            # across tiles: everything up to the later tile is absorbed; later tiles add 128
            exp_val = 128 * (N // 128 - 1 - tq)
        assert got[r] == exp_val, (p, q, got[r], exp_val)


def test_dprob_brute_force_and_offs():
    inp = W.dprob_inputs(M=9, N=300, E=3, min_tokens=1, seed=11, out_init="normal")
    offs = np.array([2, 4, 4, 7], np.int32)  # rows 0,1,7,8 untouched; one empty expert
    got = od.grouped_dprob(inp.dprob0, inp.dY, inp.C, offs)
    ref = brute.dprob(inp.dprob0, inp.dY, inp.C, offs)
    assert np.array_equal(bits(got), bits(ref))
    assert np.array_equal(bits(got[[0, 1, 7, 8]]), bits(inp.dprob0[[0, 1, 7, 8]]))


def test_dprob_invariants():
    inp = W.dprob_inputs(M=20, N=512, E=2, min_tokens=1, seed=13, out_init="normal")
    z = od.grouped_dprob(np.full(20, -0.0, np.float32), inp.dY, inp.C, inp.offs)
    full = od.grouped_dprob(inp.dprob0, inp.dY, inp.C, inp.offs)
    assert np.array_equal(bits(full), bits(inp.dprob0 + z))  # accumulate = one add of the total
    # scaling dY by 2^3 scales the result exactly
    dY8 = W.bf16_bits(widen_bf16(inp.dY) * np.float32(8))
    z8 = od.grouped_dprob(np.zeros(20, np.float32), dY8, inp.C, inp.offs)
    assert np.array_equal(z8, z * np.float32(8))
    # empty problem leaves the output bitwise unchanged
    e = od.grouped_dprob(inp.dprob0, inp.dY, inp.C, np.array([4, 4, 4], np.int32))
    assert np.array_equal(bits(e), bits(inp.dprob0))


# ----------------------------------------------------------------------- dbias
@pytest.mark.parametrize("M,N,BM", [(4096, 64, 128), (777, 33, 64), (300, 8, 256), (5, 3, 64)])
def test_dbias_fp64_bound(M, N, BM):
    inp = W.dbias_inputs(M=M, N=N, E=5, min_tokens=1, seed=17, out_init="normal")
    got = odb.grouped_dbias(inp.dbias0, inp.dA, inp.offs, BM)
    exact, absum = fp64.dbias64(inp.dbias0, inp.dA, inp.offs)
    n_tiles = max(len(t) for t in odb.tile_ranges(inp.offs, M, BM))
    d = int(np.log2(BM)) + n_tiles + 1  # tree depth + fold length + final add
    bound = gamma(d) * (absum + np.abs(inp.dbias0)) + 2.0 ** -149
    assert np.all(np.abs(got - exact) <= bound)
    assert rel_l2(got, exact) <= 1e-5


def test_dbias_exact_integers():
    inp = W.dbias_inputs(M=3000, N=40, E=6, min_tokens=1, seed=19, integer=True)
    d0 = np.random.default_rng(5).integers(-100, 100, inp.dbias0.shape).astype(np.float32)
    got = odb.grouped_dbias(d0, inp.dA, inp.offs, 128)
    x = widen_bf16(inp.dA).astype(np.int64)
    exact = d0.astype(np.int64).copy()
    for e in range(len(inp.offs) - 1):
        exact[e] += x[inp.offs[e]:inp.offs[e + 1]].sum(0)
    assert np.array_equal(got.astype(np.int64), exact)


def test_dbias_order_probe():
    """+-2^40 at two rows of one expert: the count of 1.0s absorbed reveals the
    tree inside a tile and the left fold across tiles."""
    BM, rows = 64, 640
    cases = [(0, 1), (0, 63), (5, 40), (64, 65), (10, 300), (0, 639), (200, 500)]
    N = len(cases)
    x = np.ones((rows, N), np.float32)
    for j, (p, q) in enumerate(cases):
        x[p, j], x[q, j] = 2.0 ** 40, -(2.0 ** 40)
    got = odb.grouped_dbias(np.zeros((1, N), np.float32), W.bf16_bits(x), np.array([0, rows], np.int32), BM)
    n_t = rows // BM
    for j, (p, q) in enumerate(cases):
        tp, tq = p // BM, q // BM
        if tp == tq:
            want = (BM - 2 ** int((p % BM) ^ (q % BM)).bit_length()) + BM * (n_t - 1)
        else:
            want = BM * (n_t - 1 - tq)
        assert got[0, j] == want, (p, q, got[0, j], want)


def test_dbias_brute_force_and_offsets():
    inp = W.dbias_inputs(M=50, N=5, E=4, min_tokens=1, seed=23, out_init="normal")
    for offs in (inp.offs, np.array([3, 20, 20, 9, 44], np.int32), np.array([-5, 7, 60, 2, 70], np.int32)):
        for BM in (8, 16, 64):
            got = odb.grouped_dbias(inp.dbias0, inp.dA, offs, BM)
            ref = brute.dbias(inp.dbias0, inp.dA, offs, BM)
            assert np.array_equal(bits(got), bits(ref)), (offs, BM)
    # clamped monotone bounds: an expert whose range is empty keeps its row bitwise
    got = odb.grouped_dbias(inp.dbias0, inp.dA, np.array([3, 20, 20, 9, 44], np.int32), 16)
    assert np.array_equal(bits(got[1]), bits(inp.dbias0[1]))
    assert np.array_equal(bits(got[2]), bits(inp.dbias0[2]))


def test_dbias_aligned_experts_are_absolute_m_blocks():
    """With every expert starting on a block boundary, the tiles are the absolute
    M blocks: slots from the whole matrix cut into blocks, folded per expert."""
    BM = 32
    inp = W.dbias_inputs(M=320, N=7, E=3, min_tokens=1, seed=29, out_init="normal")
    offs = np.array([0, 64, 64, 320], np.int32)
    got = odb.grouped_dbias(inp.dbias0, inp.dA, offs, BM)
    x = widen_bf16(inp.dA)
    blocks = [x[r:r + BM] for r in range(0, 320, BM)]
    slots = []
    for blk in blocks:
        v = blk.astype(np.float32)
        while v.shape[0] > 1:
            v = (v[0::2] + v[1::2]).astype(np.float32)
        slots.append(v[0])
    want = inp.dbias0.copy()
    for e, (lo, hi) in enumerate([(0, 2), (2, 2), (2, 10)]):
        if hi > lo:
            t = np.float32(-0.0) * np.ones(7, np.float32)
            for s_ in slots[lo:hi]:
                t = (t + s_).astype(np.float32)
            want[e] = (want[e] + t).astype(np.float32)
    assert np.array_equal(bits(got), bits(want))


def test_dbias_invariants():
    inp = W.dbias_inputs(M=1000, N=16, E=4, min_tokens=1, seed=31, out_init="normal")
    z = odb.grouped_dbias(np.full(inp.dbias0.shape, -0.0, np.float32), inp.dA, inp.offs, 128)
    full = odb.grouped_dbias(inp.dbias0, inp.dA, inp.offs, 128)
    assert np.array_equal(bits(full), bits(inp.dbias0 + z))  # accumulate = one add of the total
    dA8 = W.bf16_bits(widen_bf16(inp.dA) * np.float32(8))
    z8 = odb.grouped_dbias(np.zeros(inp.dbias0.shape, np.float32), dA8, inp.offs, 128)
    assert np.array_equal(z8, z * np.float32(8))
    e = odb.grouped_dbias(inp.dbias0, inp.dA, np.array([7] * 5, np.int32), 128)
    assert np.array_equal(bits(e), bits(inp.dbias0))


# ---------------------------------------------------------------------- colsum
@pytest.mark.parametrize("T,H,BT", [(4096, 16, 128), (1000, 32, 64), (333, 8, 256), (1, 4, 64)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_colsum_fp64_bound(T, H, BT, dtype):
    inp = W.gate_inputs(T, H, seed=2, out_init="normal", dtype=dtype)
    r1, r2 = oc.colsum(inp.a, inp.dg, inp.A_log, inp.dt_bias, inp.dA_log0, inp.ddt_bias0, BT)
    e1, e2, a1, a2 = fp64.colsum64(inp.a, inp.dg, inp.A_log, inp.dt_bias, inp.dA_log0, inp.ddt_bias0)
    S = -(-T // BT)
    d = int(np.log2(BT)) + S + 1
    term_err = 8 * U  # detmath (<= 3.5 ulp) plus the three products of the term
    for got, ex, ab, o in ((r1, e1, a1, inp.dA_log0), (r2, e2, a2, inp.ddt_bias0)):
        bound = (gamma(d) + term_err) * ab + gamma(1) * np.abs(o) + 1e-30
        assert np.all(np.abs(got - ex) <= bound)
        assert rel_l2(got, ex) <= 1e-5


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_colsum_brute_force(dtype):
    inp = W.gate_inputs(37, 3, seed=5, out_init="normal", dtype=dtype)
    for BT in (8, 64):
        r = oc.colsum(inp.a, inp.dg, inp.A_log, inp.dt_bias, inp.dA_log0, inp.ddt_bias0, BT)
        b = brute.colsum(inp.a, inp.dg, inp.A_log, inp.dt_bias, inp.dA_log0, inp.ddt_bias0, BT)
        assert np.array_equal(bits(r[0]), bits(b[0])) and np.array_equal(bits(r[1]), bits(b[1]))


def test_colsum_f32_inputs_with_bf16_values_match_bf16_inputs():
    """float32 inputs holding bf16-representable values must give the same bits as
    the bf16 inputs (the widening is exact), and other float32 values must not."""
    b = W.gate_inputs(300, 5, seed=6, out_init="normal")
    f = W.gate_inputs(300, 5, seed=6, out_init="normal", dtype="f32")
    rb = oc.colsum(b.a, b.dg, b.A_log, b.dt_bias, b.dA_log0, b.ddt_bias0, 64)
    rf = oc.colsum(widen_bf16(b.a), widen_bf16(b.dg), b.A_log, b.dt_bias, b.dA_log0, b.ddt_bias0, 64)
    assert np.array_equal(bits(rb[0]), bits(rf[0])) and np.array_equal(bits(rb[1]), bits(rf[1]))
    rr = oc.colsum(f.a, f.dg, f.A_log, f.dt_bias, f.dA_log0, f.ddt_bias0, 64)
    assert not np.array_equal(bits(rr[0]), bits(rb[0]))


def test_colsum_order_probe_through_dg():
    """With a constant, g is constant per head; dg = +-M / 1 probes the tree over rows."""
    T, H, BT = 512, 2, 128
    a = W.bf16_bits(np.zeros((T, H), np.float32))
    A_log = np.zeros(H, np.float32); dt = np.zeros(H, np.float32)
    dg = np.ones((T, H), np.float32)
    dg[3, 0], dg[5, 0] = 2.0 ** 40, -2.0 ** 40        # same tile, bitlen(3^5)=3 -> block 8
    dg[10, 1], dg[300, 1] = 2.0 ** 40, -2.0 ** 40     # tiles 0 and 2
    r1, _ = oc.colsum(a, W.bf16_bits(dg), A_log, dt, np.zeros(H, np.float32), np.zeros(H, np.float32), BT)
    g = float(oc.gate_terms(a[:1], W.bf16_bits(np.ones((1, H), np.float32)), A_log, dt)[0][0, 0])
    # head 0: tile 0 keeps 128 - 8 ones, tiles 1..3 add 128 each -> 120 + 384 ones of g
    # head 1: everything up to tile 2 absorbed; tile 3 adds 128 ones of g
    assert r1[0] == np.float32(np.float32(120 * g) + np.float32(384 * g)) or abs(r1[0] - 504 * g) < 1e-3
    assert abs(r1[1] - 128 * g) <= abs(128 * g) * 4 * U


def test_colsum_invariants():
    inp = W.gate_inputs(700, 8, seed=9, out_init="normal")
    z = oc.colsum(inp.a, inp.dg, inp.A_log, inp.dt_bias, np.full(8, -0.0, np.float32), np.full(8, -0.0, np.float32), 64)
    f = oc.colsum(inp.a, inp.dg, inp.A_log, inp.dt_bias, inp.dA_log0, inp.ddt_bias0, 64)
    assert np.array_equal(bits(f[0]), bits(inp.dA_log0 + z[0]))
    dg2 = W.bf16_bits(widen_bf16(inp.dg) * np.float32(0.25))
    z2 = oc.colsum(inp.a, dg2, inp.A_log, inp.dt_bias, np.zeros(8, np.float32), np.zeros(8, np.float32), 64)
    assert np.array_equal(z2[0], z[0] * np.float32(0.25)) and np.array_equal(z2[1], z[1] * np.float32(0.25))
    e = oc.colsum(inp.a[:0], inp.dg[:0], inp.A_log, inp.dt_bias, inp.dA_log0, inp.ddt_bias0, 64)
    assert np.array_equal(bits(e[0]), bits(inp.dA_log0))
    # four accumulated microbatches = the oracle applied four times
    o1, o2 = inp.dA_log0, inp.ddt_bias0
    for mb in range(4):
        sl = slice(mb * 175, (mb + 1) * 175)
        o1, o2 = oc.colsum(inp.a[sl], inp.dg[sl], inp.A_log, inp.dt_bias, o1, o2, 64)
    ex = fp64.colsum64(inp.a, inp.dg, inp.A_log, inp.dt_bias, inp.dA_log0, inp.ddt_bias0)
    assert rel_l2(o1, ex[0]) <= 1e-5


# -------------------------------------------------------------------- index_add
def _nearest_bf16_brute(x):
    """Scalar restatement: the two bf16 values around x (as float64), the
    nearer one, ties to the one with the even last significand bit."""
    out = []
    for v in np.asarray(x, np.float32):
        if np.isnan(v):
            out.append("nan")
            continue
        if np.isinf(v) or v == 0:
            out.append(float(v))
            continue
        lo = (int(np.float32(v).view(np.uint32)) >> 16) << 16
        cand = [lo, lo + 0x10000]
        # a candidate past the largest finite value stands for 2^128 in the
        # distance (IEEE overflow rounding) and is the infinity itself
        vals = [float(np.uint32(c).view(np.float32)) for c in cand]
        dist = [float(np.sign(v)) * 2.0 ** 128 if np.isinf(w) else w for w in vals]
        d = [abs(float(v) - w) for w in dist]
        if d[0] != d[1]:
            out.append(vals[0] if d[0] < d[1] else vals[1])
        else:
            out.append(vals[0] if ((cand[0] >> 16) & 1) == 0 else vals[1])
    return out


def test_narrow_bf16_round_to_nearest_even():
    rng = np.random.default_rng(3)
    u = rng.integers(0, 2**32, size=20000, dtype=np.uint64).astype(np.uint32)
    ties = (u & np.uint32(0xFFFF0000)) | np.uint32(0x8000)   # exactly halfway
    special = np.array([0, 0x80000000, 0x7F800000, 0xFF800000, 0x7FC00000, 0x7F800001, 0x00000001, 0x007FFFFF,
                        0x7F7FFFFF, 0x7F7F8000, 0x3F808000, 0x3F818000], np.uint32)
    x = np.concatenate([u, ties, special]).view(np.float32)
    got = narrow_bf16(x)
    # the library conversion (round to nearest even) on the same values
    import torch
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.all(np.isnan(widen_bf16(got[nan])))
    # brute nearest-value choice on a sample (float64 distances), incl. ties and overflow to inf
    idx = np.r_[0:400, 20000:20400, 40000:40000 + len(special)]
    br = _nearest_bf16_brute(x[idx])
    w = widen_bf16(got[idx])
    for g, b in zip(w, br):
        assert (b == "nan" and np.isnan(g)) or (g == b and np.signbit(g) == np.signbit(b))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_gate_da_is_the_derivative(dtype):
    """da against a float64 central difference of the gate in a (independent
    of the closed form), scaled by dg: within fp32 evaluation error plus the
    output rounding."""
    g = W.gate_inputs(T=300, H=6, seed=4, dtype=dtype)
    da = oc.gate_da(g.a, g.dg, g.A_log, g.dt_bias)
    daf = widen_bf16(da) if dtype == "bf16" else da
    a64 = g.a.astype(np.float64) if dtype == "f32" else widen_bf16(g.a).astype(np.float64)
    dg64 = g.dg.astype(np.float64) if dtype == "f32" else widen_bf16(g.dg).astype(np.float64)
    nA = -np.exp(g.A_log.astype(np.float64))

    def gate(a):
        return nA[None, :] * np.logaddexp(0.0, a + g.dt_bias.astype(np.float64)[None, :])
    h = 1e-5
    fd = dg64 * (gate(a64 + h) - gate(a64 - h)) / (2 * h)
    out_rel = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -23
    err = np.abs(daf - fd)
    assert np.all(err <= np.abs(fd) * (out_rel + 1e-5) + 1e-9), float((err / (np.abs(fd) + 1e-30)).max())
    # da is never of the opposite sign to -dg (the gate falls with a)
    assert np.all(daf * dg64 <= 0)


def test_gate_da_sums_to_ddt_bias_order():
    """With float32 inputs da is the unrounded ddt_bias term: its column sums in
    the canonical order give ddt_bias bit for bit."""
    g = W.gate_inputs(T=700, H=5, seed=8, dtype="f32")
    da = oc.gate_da(g.a, g.dg, g.A_log, g.dt_bias)
    _, ddt = oc.colsum(g.a, g.dg, g.A_log, g.dt_bias, np.zeros(5, np.float32), np.zeros(5, np.float32), 128)
    from oracle.primitives import pairwise, sequential, tiles
    s = sequential(pairwise(tiles(da, 128, axis=0)), axis=0)
    assert np.array_equal(bits(np.float32(0) + s), bits(ddt))


def small_index_inputs(seed=1, P=3000, n_rows=64, dim=16, pad=0.05, out_init="normal", dtype="bf16"):
    ids = W.zipf_ids(P, n_rows, 1.1, pad, seed)
    rng = np.random.default_rng(seed)
    src = rng.standard_normal((P, dim)).astype(np.float32) * np.float32(0.02)
    if dtype == "bf16":
        src = W.bf16_bits(src)
    out0 = rng.standard_normal((n_rows, dim)).astype(np.float32) if out_init == "normal" else np.zeros((n_rows, dim), np.float32)
    return ids, src, out0


@pytest.mark.parametrize("L", [1, 4, 64, 100000])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_index_add_fp64_bound(L, dtype):
    ids, src, out0 = small_index_inputs(dtype=dtype)
    got = oi.index_add(out0, ids, src, L)
    exact, absum = fp64.index_add64(out0, ids, src)
    counts = np.bincount(ids[ids >= 0], minlength=64)
    d = (np.minimum(counts, L) + -(-counts // L) + 1)[:, None]
    bound = gamma(d) * (absum + np.abs(out0)) + 1e-30
    assert np.all(np.abs(got - exact) <= bound)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_index_add_brute_force_and_literal(dtype):
    ids, src, out0 = small_index_inputs(seed=4, P=500, n_rows=16, dim=4, dtype=dtype)
    for L in (1, 3, 16):
        assert np.array_equal(bits(oi.index_add(out0, ids, src, L)), bits(brute.index_add(out0, ids, src, L)))
    z = np.zeros_like(out0)
    # L >= longest run reproduces the literal one-row-at-a-time fold from +0
    assert np.array_equal(bits(oi.index_add(z, ids, src, 10 ** 6)), bits(brute.literal_sequential_index_add(z, ids, src)))


def test_index_add_exact_integers_and_stable_order():
    rng = np.random.default_rng(8)
    P, n_rows, D = 20000, 50, 8
    ids = W.zipf_ids(P, n_rows, 1.1, 0.05, 8)
    ids[::97] = 123456  # out of range: dropped
    k = rng.integers(-8, 9, (P, D))
    src = W.bf16_bits((k / 256.0).astype(np.float32))
    out0 = (rng.integers(-100, 100, (n_rows, D)) / 256.0).astype(np.float32)
    got = oi.index_add(out0, ids, src, 64)
    ok = (ids >= 0) & (ids < n_rows)
    exact = (out0 * 256).astype(np.int64)
    np.add.at(exact, ids[ok], k[ok])
    assert np.array_equal((got * 256).astype(np.int64), exact)
    perm, counts = oi.stable_order(ids, n_rows)
    assert np.array_equal(perm, np.nonzero(ok)[0][np.argsort(ids[ok], kind="stable")])
    # stable: inside each run, ascending source position
    keys = ids[perm]
    assert np.all((np.diff(keys) > 0) | ((np.diff(keys) == 0) & (np.diff(perm) > 0)))


def test_index_add_invariants():
    ids, src, out0 = small_index_inputs(seed=6)
    full = oi.index_add(out0, ids, src, 32)
    z = oi.index_add(np.full_like(out0, -0.0), ids, src, 32)
    touched = np.bincount(ids[ids >= 0], minlength=64) > 0
    assert np.array_equal(bits(full[touched]), bits(out0[touched] + z[touched]))
    assert np.array_equal(bits(full[~touched]), bits(out0[~touched]))
    keep = ids >= 0
    compact = oi.index_add(out0, ids[keep], src[keep], 32)
    assert np.array_equal(bits(compact), bits(full))
    none = oi.index_add(out0, np.full(10, -1, np.int32), src[:10], 32)
    assert np.array_equal(bits(none), bits(out0))


# ------------------------------------------------------------------------ wgrad
def test_wgrad_split_ranges():
    offs = np.array([0, 1024, 1024, 2600, 2601], np.int32)
    assert ow.split_ranges(offs, 512, 0) == [[(0, 1024)], [], [(1024, 2600)], [(2600, 2601)]]
    assert ow.split_ranges(offs, 512, 1) == [[(0, 512), (512, 1024)], [], [(1024, 1536), (1536, 2048), (2048, 2560),
                                                                          (2560, 2600)], [(2600, 2601)]]
    assert ow.split_ranges(offs, 512, 2)[2] == [(1024, 2048), (2048, 2600)]


def test_wgrad_exact_integers_brute():
    inp = W.wgrad_inputs(E=3, M=5, N=4, tokens=[7, 0, 40], seed=2, integer=True, out_init="normal")
    for C in (0, 1):
        got = ow.grouped_wgrad_acc(inp.main_grad0, inp.G, inp.X, inp.offs, 16, C)
        ref = brute.wgrad_exact_integer(inp.main_grad0, inp.G, inp.X, inp.offs)
        assert np.array_equal(bits(got), bits(ref))
        assert np.array_equal(bits(got[1]), bits(inp.main_grad0[1]))  # empty expert untouched


def test_wgrad_fold_order_probe():
    M_ = np.float32(2.0 ** 40)
    mg = np.zeros((1, 1), np.float32)
    parts = [np.ones((1, 1), np.float32) for _ in range(6)]
    parts[1][0, 0], parts[3][0, 0] = M_, -M_
    assert ow.fold_partials(mg, parts)[0, 0] == 2.0  # only the two after the cancellation survive


def test_wgrad_fp64_rel_l2():
    inp = W.wgrad_inputs(E=2, M=64, N=48, tokens=[600, 1100], seed=4, out_init="normal")
    got = ow.grouped_wgrad_acc(inp.main_grad0, inp.G, inp.X, inp.offs, 512, 1)
    ex = fp64.wgrad64(inp.main_grad0, inp.G, inp.X, inp.offs)
    assert rel_l2(got, ex) <= 1e-5


def test_wgrad_bf16_accumulate_is_the_bf16_tensor_add():
    """The bf16 accumulate equals a bf16 tensor add of the bf16-rounded dW (the
    library's AccumulateGrad for a bf16 gradient), including exponent gaps,
    ties, signed zeros and overflow."""
    import torch
    rng = np.random.default_rng(11)
    n = 50000
    mg = narrow_bf16((rng.standard_normal(n) * np.exp2(rng.integers(-30, 30, n))).astype(np.float32))
    dW = (rng.standard_normal(n) * np.exp2(rng.integers(-40, 40, n))).astype(np.float32)
    mg[:4] = narrow_bf16(np.array([0.0, -0.0, 3.0e38, -0.0], np.float32))
    dW[:4] = np.array([-0.0, -0.0, 3.0e38, 0.0], np.float32)
    got = ow.accumulate_bf16(mg, dW)
    t = torch.from_numpy(mg.view(np.int16).copy()).view(torch.bfloat16)
    t.add_(torch.from_numpy(dW).to(torch.bfloat16))
    assert np.array_equal(got, t.view(torch.int16).numpy().view(np.uint16))


def test_wgrad_bf16_exact_integers_and_empty_expert():
    """Small integer inputs: dW and main_grad + dW are integers bf16 holds
    exactly, so the bf16 result is the exact sum; an empty expert keeps its bits."""
    inp = W.wgrad_inputs(E=3, M=16, N=24, tokens=[40, 0, 700], integer=True, seed=2)
    mg0 = narrow_bf16(np.random.default_rng(4).integers(-8, 9, size=(3, 16, 24)).astype(np.float32))
    for C in (0, 1):
        got = ow.grouped_wgrad_acc_bf16(mg0, inp.G, inp.X, inp.offs, ktiles_per_split=C)
        Gf, Xf = widen_bf16(inp.G).astype(np.float64), widen_bf16(inp.X).astype(np.float64)
        o = inp.offs
        for e in range(3):
            exact = widen_bf16(mg0[e]).astype(np.float64) + Gf[o[e]:o[e + 1]].T @ Xf[o[e]:o[e + 1]]
            assert np.all(np.abs(exact) <= 256)
            if o[e + 1] == o[e]:
                assert np.array_equal(got[e], mg0[e])
            else:
                assert np.array_equal(widen_bf16(got[e]).astype(np.float64), exact)
