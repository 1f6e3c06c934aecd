"""Pins of the float32 detmath sequences against float64 libm (CPU).

The sequences are fixed so that two independent implementations agree
bitwise; these tests pin them to the mathematics: every result stays within a
small ulp bound of the float64 value over dense samples of the domain that the
gate backward uses, and the special values come out as IEEE-754 defines them.
A wrong coefficient, reduction constant or branch moves results by many ulps.
Measured maxima on 3-4 M samples: exp32 1.19, log1p32 1.90, softplus32 2.73,
sigmoid32 2.31 ulp; the bounds below add a margin.
"""
import numpy as np
import pytest

from oracle import detmath as dm

RNG = np.random.default_rng(1234)


def ulp_err(r, exact):
    ex32 = exact.astype(np.float32)
    ulp = np.maximum(np.spacing(np.abs(ex32)).astype(np.float64), 2.0 ** -149)
    return np.abs(r.astype(np.float64) - exact) / ulp


def test_exp32_ulp():
    x = np.concatenate([RNG.uniform(-104, 88.72, 1_000_000), RNG.uniform(-1, 1, 300_000),
                        RNG.uniform(-25, 0, 300_000)]).astype(np.float32)
    with np.errstate(all="ignore"):
        e = ulp_err(dm.exp32(x), np.exp(x.astype(np.float64)))
    assert e.max() <= 1.5


def test_exp32_special_values():
    f = np.float32
    assert dm.exp32(f(0.0)) == 1.0 and dm.exp32(f(-0.0)) == 1.0
    assert dm.exp32(f(np.inf)) == np.inf and dm.exp32(f(-np.inf)) == 0.0
    assert np.isnan(dm.exp32(f(np.nan)))
    assert dm.exp32(f(89.5)) == np.inf and dm.exp32(f(-105.0)) == 0.0
    # exact powers: exp(k ln2) is 2^k up to the reduction error of k*ln2 in float32
    assert dm.exp32(f(1.0)) == f(np.e)
    # subnormal results: within one subnormal quantum
    x = np.float32(-100.0)
    assert abs(float(dm.exp32(x)) - np.exp(-100.0)) <= 2.0 ** -149
    # monotone on a dense grid
    g = np.linspace(-30, 30, 200001).astype(np.float32)
    assert np.all(np.diff(dm.exp32(g).astype(np.float64)) >= 0)


def test_log1p32_ulp():
    y = np.concatenate([RNG.uniform(0, 1, 1_000_000), np.exp2(-RNG.uniform(0, 140, 100_000))]).astype(np.float32)
    assert ulp_err(dm.log1p32(y), np.log1p(y.astype(np.float64))).max() <= 2.5
    assert dm.log1p32(np.float32(0.0)) == 0.0
    assert dm.log1p32(np.float32(1.0)) == np.float32(np.log(2.0)) or \
        abs(float(dm.log1p32(np.float32(1.0))) - np.log(2.0)) <= 2 * 2.0 ** -24


def test_softplus32_ulp_and_threshold():
    x = np.concatenate([RNG.uniform(-100, 100, 1_000_000), RNG.uniform(-25, 25, 1_000_000)]).astype(np.float32)
    x64 = x.astype(np.float64)
    ref = np.where(x64 > 20, x64, np.logaddexp(0.0, x64))
    assert ulp_err(dm.softplus32(x), ref).max() <= 3.5
    big = np.array([20.000002, 21.0, 1e30, np.inf], np.float32)
    assert np.array_equal(dm.softplus32(big), big)
    assert dm.softplus32(np.float32(-200.0)) == 0.0
    assert np.isnan(dm.softplus32(np.float32(np.nan)))


def test_sigmoid32_ulp_and_symmetry():
    x = np.concatenate([RNG.uniform(-100, 100, 1_000_000), RNG.uniform(-10, 10, 1_000_000)]).astype(np.float32)
    ref = 1.0 / (1.0 + np.exp(-x.astype(np.float64)))
    assert ulp_err(dm.sigmoid32(x), ref).max() <= 3.0
    assert dm.sigmoid32(np.float32(0.0)) == 0.5 and dm.sigmoid32(np.float32(-0.0)) == 0.5
    assert dm.sigmoid32(np.float32(200.0)) == 1.0 and dm.sigmoid32(np.float32(-200.0)) == 0.0


def test_shared_e_forms_equal_standalone():
    x = RNG.uniform(-30, 30, 10000).astype(np.float32)
    e = dm.exp32(-np.abs(x))
    assert np.array_equal(dm.softplus_from(x, e).view(np.uint32), dm.softplus32(x).view(np.uint32))
    assert np.array_equal(dm.sigmoid_from(x, e).view(np.uint32), dm.sigmoid32(x).view(np.uint32))


@pytest.mark.parametrize("fn", ["exp32", "log1p32"])
def test_no_fused_ops_in_reference_sequence(fn):
    """A fused multiply-add changes the bits of a few percent of results.

    Re-evaluating the Horner steps with float64 products (a stand-in for a
    fused multiply-add) must differ somewhere, which shows the pins above are
    sensitive to the one-rounding-per-operation rule.
    """
    x = RNG.uniform(-10, 0, 20000).astype(np.float32) if fn == "exp32" else RNG.uniform(0, 1, 20000).astype(np.float32)
    ref = getattr(dm, fn)(x)
    if fn == "exp32":
        kf = np.rint(x * dm.INV_LN2).astype(np.float32)
        r = ((x - kf * dm.LN2_HI) - kf * dm.LN2_LO).astype(np.float32)
        p = np.full(x.shape, dm.EXP_C[7], np.float64)
        for c in dm.EXP_C[6::-1]:
            p = (p * r.astype(np.float64) + np.float64(c)).astype(np.float32).astype(np.float64)
        k = kf.astype(np.int64)
        fused = (p.astype(np.float32) * dm._pow2(k >> 1)) * dm._pow2(k - (k >> 1))
    else:
        s = (x / (np.float32(2) + x)).astype(np.float32)
        z = (s * s).astype(np.float32)
        q = np.full(x.shape, dm.LOG_D[13], np.float64)
        for i in (11, 9, 7, 5, 3):
            q = (q * z + np.float64(dm.LOG_D[i])).astype(np.float32).astype(np.float64)
        q = (q * z).astype(np.float32)
        t = s + s
        fused = (t.astype(np.float64) + t.astype(np.float64) * q).astype(np.float32)
    assert not np.array_equal(fused.view(np.uint32), ref.view(np.uint32))
