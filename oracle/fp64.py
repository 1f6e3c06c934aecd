"""Exact definitions in float64, used only to pin the float32 oracle (test infrastructure).

Each function is the plain mathematical statement of one case with no
attention to order: float64 sums of exactly widened inputs. Float64 carries 29
more significand bits than float32, so these values serve as the "exact" side
of error bounds (Higham, Accuracy and Stability of Numerical Algorithms, ch. 4).
The transcendental functions here are numpy's float64 ones, independent of the
float32 detmath sequences.
"""
from __future__ import annotations

import numpy as np


def widen(bits) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def gate_terms64(a_bits, dg_bits, A_log, dt_bias):
    a = np.asarray(a_bits, np.float64) if np.asarray(a_bits).dtype == np.float32 else widen(a_bits)
    dg = np.asarray(dg_bits, np.float64) if np.asarray(dg_bits).dtype == np.float32 else widen(dg_bits)
    x = a + np.asarray(dt_bias, np.float64)[None, :]
    nA = -np.exp(np.asarray(A_log, np.float64))[None, :]
    sp = np.where(x > 20.0, x, np.logaddexp(0.0, x))
    sg = 1.0 / (1.0 + np.exp(-x))
    return dg * nA * sp, dg * nA * sg


def colsum64(a_bits, dg_bits, A_log, dt_bias, dA0, ddt0):
    t1, t2 = gate_terms64(a_bits, dg_bits, A_log, dt_bias)
    return np.asarray(dA0, np.float64) + t1.sum(0), np.asarray(ddt0, np.float64) + t2.sum(0), \
        np.abs(t1).sum(0), np.abs(t2).sum(0)


def dprob64(dprob0, dY_bits, C_bits, offs):
    M = len(dprob0)
    lo = int(min(max(offs[0], 0), M)); hi = int(min(max(offs[-1], lo), M))
    y = widen(dY_bits[lo:hi]); c = widen(C_bits[lo:hi])
    term = y * np.maximum(c, 0.0) ** 2
    out = np.asarray(dprob0, np.float64).copy()
    out[lo:hi] += term.sum(1)
    absum = np.zeros(M); absum[lo:hi] = np.abs(term).sum(1)
    return out, absum


def index_add64(out0, ids, src_bits):
    out = np.asarray(out0, np.float64).copy()
    ids = np.asarray(ids, np.int64)
    ok = (ids >= 0) & (ids < out.shape[0])
    sb = np.asarray(src_bits)[ok]
    src = sb.astype(np.float64) if sb.dtype == np.float32 else widen(sb)
    absum = np.zeros_like(out)
    np.add.at(out, ids[ok], src)
    np.add.at(absum, ids[ok], np.abs(src))
    return out, absum


def wgrad64(main_grad0, G_bits, X_bits, offs, experts=None):
    out = np.asarray(main_grad0, np.float64).copy()
    for e in range(len(offs) - 1):
        if experts is not None and e not in experts:
            continue
        lo, hi = int(offs[e]), int(offs[e + 1])
        if hi > lo:
            out[e] += widen(G_bits[lo:hi]).T @ widen(X_bits[lo:hi])
    return out


def dbias64(dbias0, dA_bits, offs):
    out = np.asarray(dbias0, np.float64).copy()
    absum = np.zeros_like(out)
    M = dA_bits.shape[0]
    prev = 0
    b = []
    for e, o in enumerate(np.asarray(offs, np.int64)):
        v = int(min(max(int(o), 0 if e == 0 else prev), M)); b.append(v); prev = v
    for e in range(len(b) - 1):
        x = widen(dA_bits[b[e]:b[e + 1]])
        out[e] += x.sum(0)
        absum[e] = np.abs(x).sum(0)
    return out, absum
