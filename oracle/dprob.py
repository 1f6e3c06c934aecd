"""Grouped-GEMM dsReLU backward dprob with per-N-tile slots (test infrastructure only).

cudnn-frontend PR #521 (deterministic dprob in the grouped-GEMM dsReLU
backward), first commit: dprob, a float sum over n, varied from run to run
both inside a CTA (the order of its N subtiles) and across CTAs (atomics on the
same token). The fix stores each subtile's partial in its own slot, addressed
by which subtile it is, allots dprob one slot per N tile so that no slot has
two writers, folds the slots in one fixed order and adds the result to the
existing dprob.

    dprob[m] += sum_n dY[m, n] * srelu(C[m, n]),   srelu(c) = relu(c)^2

Canonical order: term = f32(dY) * sq with sq = c*c if c > 0 else +0.0 (the
product has at most 8+8+8 significand bits, so it is exact whenever it is a
normal number); one slot per 128-wide N tile holding the adjacent pairwise tree
of its 128 terms (columns past N are -0.0); the slots folded left to right in
tile order; one add into dprob[m].

Rows are grouped by expert (``offs``, E+1 row offsets). Rows are independent,
so the grouping changes nothing except which rows are valid: rows outside
[offs[0], offs[E]) are left untouched (the valid_m rows of the page's dprob
tensor).
"""
from __future__ import annotations

import numpy as np

from .primitives import accumulate, pairwise, sequential, tiles, widen_bf16

TILE_N = 128


def dprob_terms(dY_bits, C_bits) -> np.ndarray:
    y = widen_bf16(dY_bits)
    c = widen_bf16(C_bits)
    sq = np.where(c > np.float32(0.0), c * c, np.float32(0.0)).astype(np.float32)
    return (y * sq).astype(np.float32)


def dprob_slots(dY_bits, C_bits, tile_n: int = TILE_N) -> np.ndarray:
    """[rows, ceil(N/tile_n)] slot matrix."""
    return pairwise(tiles(dprob_terms(dY_bits, C_bits), tile_n, axis=1))


def valid_rows(offs, M: int):
    offs = np.asarray(offs, np.int64)
    lo = int(min(max(offs[0], 0), M))
    hi = int(min(max(offs[-1], lo), M))
    return lo, hi


def grouped_dprob(dprob0, dY_bits, C_bits, offs, tile_n: int = TILE_N) -> np.ndarray:
    dprob0 = np.asarray(dprob0, np.float32)
    M = dprob0.shape[0]
    lo, hi = valid_rows(offs, M)
    out = dprob0.copy()
    if hi > lo:
        total = sequential(dprob_slots(dY_bits[lo:hi], C_bits[lo:hi], tile_n), axis=1)
        out[lo:hi] = accumulate(out[lo:hi], total)
    return out
