"""Fused sparse-indexer dK: the index_add of source rows made on the fly from the
clipped-KL score gradient (test infrastructure only).

Megatron-LM PR #7441 (DSv4 deterministic mode), source 3 and its fix: the
deterministic indexer backward computes the same clipped-log KL gradient as the
cuDNN kernel, the score gradient predict * sum(kept_target) - kept_target with
the targets clamped at e^-100 and a valid-slot mask, normalised by
loss_coeff / (B * S_q) * sm_scale * grad_loss, and accumulates dK over the
per-sample key ids without atomics (stable sort + prefix sum).

Readings taken here (the page names the terms, not a formula text):
* Per query row r and top-k slot j, a slot is valid when its id lies in
  [0, n_rows); padding (-1) and any other out-of-range id are dropped.
* kept_j = max(target_j, EPS) on a valid slot and 0 on a dropped one, with
  EPS = RN32(e^-100) = 27 * 2^-149 (a subnormal float32).
* S_r = the left-to-right float32 sum of kept_j over the row's slots in slot
  order, from -0.0 (the canonical top-k order, when the caller passes ids and
  predict from the canonical top-k).
* g_j = RN32(RN32(predict_j * S_r) - kept_j) and the slot coefficient
  c_j = RN32(g_j * scale), where scale is the caller's float32 product
  loss_coeff / (B * S_q) * sm_scale * grad_loss (the indexer score being
  sm_scale * q . k, its gradient with respect to k is sm_scale * q).
* The source row of slot (r, j) is src[d] = RN32(c_j * q[r][d]) (q widened
  exactly from bf16); dK += the canonical index_add of these rows over the ids
  (stable id order, chunks of L rows, oracle/index_add.py).
"""
from __future__ import annotations

import numpy as np

from . import index_add as oi
from .primitives import NEG_ZERO, widen_bf16

EPS_BITS = 0x0000001B  # RN32(e^-100): e^-100 / 2^-149 = 26.55, rounded to 27


def eps() -> np.float32:
    return np.array([EPS_BITS], np.uint32).view(np.float32)[0]


def valid_mask(ids, n_rows: int) -> np.ndarray:
    ids = np.asarray(ids, np.int64)
    return (ids >= 0) & (ids < n_rows)


def kept_targets(ids, target, n_rows: int) -> np.ndarray:
    """kept[r, j] = max(target, EPS) on valid slots, +0 elsewhere."""
    t = np.asarray(target, np.float32)
    return np.where(valid_mask(ids, n_rows), np.maximum(t, eps()), np.float32(0.0)).astype(np.float32)


def row_sums(kept: np.ndarray) -> np.ndarray:
    """S[r] = ((-0 + kept[r, 0]) + kept[r, 1]) + ... in slot order."""
    S = np.full(kept.shape[0], NEG_ZERO, np.float32)
    for j in range(kept.shape[1]):
        S = np.add(S, kept[:, j], dtype=np.float32)
    return S


def coefficients(ids, predict, target, n_rows: int, scale) -> np.ndarray:
    """c[r, j] = RN32(RN32(RN32(predict * S_r) - kept) * scale) on valid slots (0 on dropped ones)."""
    kept = kept_targets(ids, target, n_rows)
    S = row_sums(kept)
    p = np.asarray(predict, np.float32)
    g = np.subtract(np.multiply(p, S[:, None], dtype=np.float32), kept, dtype=np.float32)
    c = np.multiply(g, np.float32(scale), dtype=np.float32)
    return np.where(valid_mask(ids, n_rows), c, np.float32(0.0)).astype(np.float32)


def source_rows(coef: np.ndarray, q_bits) -> np.ndarray:
    """src[(r, j), d] = RN32(c[r, j] * q[r, d]), [Q * K, D] float32, row-major over (r, j)."""
    q = np.asarray(q_bits)
    q = q.astype(np.float32) if q.dtype == np.float32 else widen_bf16(q)
    Q, K = coef.shape
    return np.multiply(coef[:, :, None], q[:, None, :], dtype=np.float32).reshape(Q * K, q.shape[1])


def indexer_dk(dk0, ids, predict, target, q_bits, scale, chunk_rows: int) -> np.ndarray:
    """dK after the fused accumulation (dk0 [n_rows, D] float32 is not modified).

    ids, predict, target: [Q, K]; q_bits: [Q, D] bf16 bits (or float32 values)."""
    n_rows = np.asarray(dk0).shape[0]
    coef = coefficients(ids, predict, target, n_rows, scale)
    src = source_rows(coef, q_bits)
    return oi.index_add(dk0, np.asarray(ids).reshape(-1), src, chunk_rows)
