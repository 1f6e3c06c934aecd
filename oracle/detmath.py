"""Bit-reproducible float32 exp, log1p, softplus and sigmoid (test infrastructure only).

The gate backward (Megatron-LM PR #8244) needs exp, softplus and sigmoid. The
pages do not say how they are evaluated, and a hardware approximate
instruction has no published bit pattern, so a CPU oracle could never agree
with it bit for bit. The reading taken here: each function is a fixed
sequence of correctly rounded binary32 operations (+, -, *, / with
round-to-nearest-even, no fused multiply-add) plus exact operations (sign and
exponent bit manipulation, round-to-nearest-even to an integer, comparisons).
Any two implementations of the same sequence then agree bitwise.

exp32(x)
    NaN -> NaN; x > 89 -> +inf; x < -104 -> +0. Otherwise Cody-Waite
    reduction: k = rint(x * INV_LN2) with INV_LN2 = RN32(1/ln 2)
    (bits 0x3FB8AA3B); r = (x - k*LN2_HI) - k*LN2_LO with LN2_HI = 0x3F317200
    (16 significant bits, so k*LN2_HI is exact for |k| <= 255) and
    LN2_LO = 0x35BFBE8E. p = Taylor polynomial of degree 7 in Horner form,
    coefficients c_i = RN32(1 / i!) (c0 = c1 = 1): p = c7; p = p*r + c6; ...;
    p = p*r + c0, each step one multiply then one add. The result is
    p * 2^k1 * 2^k2 (two multiplies, left to right) with k1 = floor(k / 2),
    k2 = k - k1, so only the second multiply can round (subnormal results) or
    overflow.
log1p32(y), y >= 0 (used on [0, 1])
    s = y / (2 + y); z = s*s; q = d13; q = q*z + d11; q = q*z + d9;
    q = q*z + d7; q = q*z + d5; q = q*z + d3; q = q*z with d_i = RN32(1/i);
    t = s + s; result = t + t*q. This is the series log1p(y) = 2 atanh(y/(2+y))
    truncated after the s^13 term (truncation below 2^-26 relative on [0, 1]).
softplus32(x)
    x > 20 -> x (the threshold PyTorch's softplus uses by default; the pages are
    silent). Otherwise m + log1p32(exp32(-|x|)) with m = x if x > 0 else +0.
sigmoid32(x)
    e = exp32(-|x|); (1 if x >= 0 else e) / (1 + e).
"""
from __future__ import annotations

import numpy as np

F32 = np.float32


def _bits(b: int) -> np.float32:
    return np.array([b], np.uint32).view(np.float32)[0]


INV_LN2 = _bits(0x3FB8AA3B)
LN2_HI = _bits(0x3F317200)
LN2_LO = _bits(0x35BFBE8E)
ONE = F32(1.0)
TWO = F32(2.0)
ZERO = F32(0.0)
# Taylor coefficients RN32(1/i!) for i = 0..7, each one correctly rounded division.
_FACT = [1, 1, 2, 6, 24, 120, 720, 5040]
EXP_C = [F32(1.0) / F32(f) for f in _FACT]
# atanh-series coefficients RN32(1/i) for i = 3, 5, ..., 13.
LOG_D = {i: F32(1.0) / F32(i) for i in (3, 5, 7, 9, 11, 13)}


def _pow2(n: np.ndarray) -> np.ndarray:
    """2^n as float32 for integer n in [-126, 127], built from exponent bits."""
    return ((n.astype(np.int64) + 127) << 23).astype(np.uint32).view(np.float32)


def exp32(x) -> np.ndarray:
    x = np.asarray(x, np.float32)
    with np.errstate(over="ignore", invalid="ignore", under="ignore"):
        big = x > F32(89.0)
        small = x < F32(-104.0)
        nan = np.isnan(x)
        xs = np.where(big | small | nan, ZERO, x).astype(np.float32)
        kf = np.rint(xs * INV_LN2).astype(np.float32)
        r = (xs - kf * LN2_HI) - kf * LN2_LO
        p = EXP_C[7]
        for c in (EXP_C[6], EXP_C[5], EXP_C[4], EXP_C[3], EXP_C[2], EXP_C[1], EXP_C[0]):
            p = p * r
            p = p + c
        k = kf.astype(np.int64)
        k1 = k >> 1
        k2 = k - k1
        res = (p * _pow2(k1)) * _pow2(k2)
        res = np.where(big, F32(np.inf), res)
        res = np.where(small, ZERO, res)
        res = np.where(nan, x, res)
    return res.astype(np.float32)


def log1p32(y) -> np.ndarray:
    y = np.asarray(y, np.float32)
    with np.errstate(over="ignore", invalid="ignore", under="ignore"):
        s = y / (TWO + y)
        z = s * s
        q = np.full(y.shape, LOG_D[13], np.float32)
        for i in (11, 9, 7, 5, 3):
            q = q * z
            q = q + LOG_D[i]
        q = q * z
        t = s + s
        return (t + t * q).astype(np.float32)


def softplus_from(x: np.ndarray, e: np.ndarray) -> np.ndarray:
    """softplus32(x) given e = exp32(-|x|)."""
    m = np.where(x > ZERO, x, ZERO).astype(np.float32)
    small = m + log1p32(e)
    return np.where(x > F32(20.0), x, small).astype(np.float32)


def sigmoid_from(x: np.ndarray, e: np.ndarray) -> np.ndarray:
    """sigmoid32(x) given e = exp32(-|x|)."""
    with np.errstate(invalid="ignore"):
        num = np.where(x >= ZERO, ONE, e).astype(np.float32)
        return (num / (ONE + e)).astype(np.float32)


def neg_abs_exp(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, np.float32)
    return exp32(-np.abs(x))


def softplus32(x) -> np.ndarray:
    x = np.asarray(x, np.float32)
    return softplus_from(x, neg_abs_exp(x))


def sigmoid32(x) -> np.ndarray:
    x = np.asarray(x, np.float32)
    return sigmoid_from(x, neg_abs_exp(x))
