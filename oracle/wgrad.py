"""Grouped weight gradient with fixed-order split-K accumulation (test infrastructure only).

FlashInfer PR #8602 (fuse the fp32 weight-gradient accumulate into main_grad)
and its follow-up #8924 (deterministic weight-gradient accumulation):

    main_grad[e] += G_e^T X_e,   G_e = G[o_e:o_{e+1}],  X_e = X[o_e:o_{e+1}]

with expert offsets read on the device. The deterministic route's result is
bitwise the AccumulateGrad of the deterministic dW, i.e. RN32(main_grad + dW)
with dW computed in a fixed order (#8924 summary, item 3).

Canonical order (the reading taken here):
* The token rows of expert e are cut into K tiles of ``k_tile`` (512) rows
  counted from the expert's first row; ``ktiles_per_split`` consecutive K tiles
  form one split (0 means the whole expert is one split).
* Each split s produces a float32 partial Q_s[i, j] by a chain of matrix-core
  steps over its rows in ascending 16-row blocks, starting from +0.0. The
  steps' own rounding is a property of the matrix-core instruction, which the
  pages do not describe; ``chain_mfma`` takes it from the instruction model of
  oracle/mfma.py (the default), and ``chain_exact_rounded`` is the exact
  product rounded once, which every order gives when all partial sums are
  exactly representable (small-integer inputs).
* main_grad[e][i, j] <- RN32(main_grad[e][i, j] + fold(Q_0 .. Q_{S_e - 1}))
  with fold the left-to-right sum starting at -0.0. An expert with no rows
  leaves its main_grad slice bitwise unchanged.
* A bf16 main_grad (#8924, "Design and numerics": for bf16 out the bf16 dW is
  added in bf16, bitwise the AccumulateGrad of the deterministic dW): the same
  fold gives the float32 dW, which is rounded to bf16 (nearest even); the two
  bf16 values are added in float32 (RN32) and the sum rounded to bf16, as a
  bf16 tensor add does.
"""
from __future__ import annotations

import numpy as np

from . import mfma
from .primitives import NEG_ZERO, accumulate, narrow_bf16, widen_bf16

K_TILE = 512


def split_ranges(offs, k_tile: int = K_TILE, ktiles_per_split: int = 0):
    """Per expert, the list of (row_begin, row_end) of its splits."""
    offs = np.asarray(offs, np.int64)
    out = []
    for e in range(len(offs) - 1):
        lo, hi = int(offs[e]), int(offs[e + 1])
        if hi <= lo:
            out.append([])
            continue
        step = (hi - lo) if ktiles_per_split <= 0 else k_tile * ktiles_per_split
        out.append([(b, min(b + step, hi)) for b in range(lo, hi, step)])
    return out


def fold_total(partials, shape) -> np.ndarray:
    """Left-to-right fold of the partial list, from -0.0."""
    total = np.full(shape, NEG_ZERO, np.float32)
    for q in partials:
        total = np.add(total, np.asarray(q, np.float32), dtype=np.float32)
    return total


def fold_partials(main_grad0: np.ndarray, partials) -> np.ndarray:
    """RN32(main_grad0 + left-to-right fold of the partial list)."""
    return accumulate(main_grad0, fold_total(partials, main_grad0.shape))


def accumulate_bf16(main_grad_bits: np.ndarray, dW: np.ndarray) -> np.ndarray:
    """bf16 main_grad (uint16 bits) plus the float32 dW, added in bf16:
    RN_bf16(RN32(main_grad + RN_bf16(dW)))."""
    d16 = widen_bf16(narrow_bf16(dW))
    return narrow_bf16(np.add(widen_bf16(main_grad_bits), d16, dtype=np.float32))


def chain_mfma(G_bits: np.ndarray, X_bits: np.ndarray, r0: int, r1: int, rows=None) -> np.ndarray:
    """Q over token rows [r0, r1) of G [T, M] and X [T, N] (bf16 bits): per output (i, j) the chain of
    the matrix-core step model from +0 over 16-row blocks counted from r0 (rows past r1 are zero), for
    the output rows ``rows`` (all by default)."""
    return mfma.wgrad_partial(G_bits, X_bits, r0, r1, rows)


def chain_exact_rounded(G_bits: np.ndarray, X_bits: np.ndarray, r0: int, r1: int, rows=None) -> np.ndarray:
    """RN32 of the exact G^T X over rows [r0, r1) (float64 is exact for small-integer inputs).

    Any summation order gives this result whenever every partial sum is an
    exactly representable integer, so it is the chain for exact-integer pins.
    """
    g = widen_bf16(G_bits[r0:r1]).astype(np.float64)
    if rows is not None:
        g = g[:, np.asarray(rows)]
    return (g.T @ widen_bf16(X_bits[r0:r1]).astype(np.float64)).astype(np.float32)


def grouped_wgrad_acc(main_grad0, G_bits, X_bits, offs, k_tile: int = K_TILE, ktiles_per_split: int = 0,
                      chain=chain_mfma, experts=None, rows=None) -> np.ndarray:
    """Return the updated main_grad [E, M, N] (main_grad0 is not modified).

    With ``rows`` (output row indices), only those rows are computed and the
    result is [E, len(rows), N]; with ``experts``, other experts keep main_grad0."""
    mg = np.array(main_grad0 if rows is None else np.asarray(main_grad0)[:, np.asarray(rows)], np.float32, copy=True)
    splits = split_ranges(offs, k_tile, ktiles_per_split)
    for e, sp in enumerate(splits):
        if experts is not None and e not in experts:
            continue
        if not sp:
            continue
        parts = [chain(G_bits, X_bits, b, t, rows) for b, t in sp]
        mg[e] = fold_partials(mg[e], parts)
    return mg


def grouped_wgrad_acc_bf16(main_grad0_bits, G_bits, X_bits, offs, k_tile: int = K_TILE, ktiles_per_split: int = 0,
                           chain=chain_mfma, experts=None, rows=None) -> np.ndarray:
    """bf16 main_grad [E, M, N] (uint16 bits) after the bf16 accumulate of the
    deterministic dW; experts with no rows keep their bits. ``rows`` as for
    grouped_wgrad_acc."""
    mg0 = np.asarray(main_grad0_bits)
    mg = np.array(mg0 if rows is None else mg0[:, np.asarray(rows)], np.uint16, copy=True)
    splits = split_ranges(offs, k_tile, ktiles_per_split)
    for e, sp in enumerate(splits):
        if (experts is not None and e not in experts) or not sp:
            continue
        parts = [chain(G_bits, X_bits, b, t, rows) for b, t in sp]
        mg[e] = accumulate_bf16(mg[e], fold_total(parts, mg[e].shape))
    return mg
