"""Canonical compact top-k: per-row id order and the softmax recomputed in it
(test infrastructure only).

Megatron-LM PR #7441 (DSv4 deterministic mode), source 1 and its fix: the
order in which a row's selected ids (and the terms of its softmax sum) come
out varied between runs; the fix puts every row in one canonical order, with
the padding at the end and the logits moved alongside, sums the softmax again
in that order, and leaves rows without a valid id at probability zero.

Canonical definition (the reading taken here), per row q of K slots:
* order: the slots with a valid id (>= 0) by ascending id, equal ids by
  ascending slot; then the padding slots (negative ids) by ascending slot;
* ids_out and logits_out are ids and logits in that order;
* m = the largest logit of the valid slots (exact in any order);
  e_j = exp32(logit_j - m) for valid slots (exp32 as in the gate's detmath);
  S = the left-to-right sum of the e_j in the new order, from -0.0;
  probs_out_j = e_j / S for valid slots (one correctly rounded division),
  +0.0 for padding; a row with no valid slot has all probabilities +0.0.
The ids, the probabilities and the logits of valid slots depend only on the
multiset of (id, logit) pairs per row (up to the order of equal ids), so a
run-dependent slot order of distinct ids cannot change a bit of them; padding
slots keep their logits in slot order (the page permutes all logits with the
same permutation).
"""
from __future__ import annotations

import numpy as np

from . import detmath


def canonical_order(ids_row: np.ndarray) -> np.ndarray:
    """Slot permutation of one row: valid ids ascending (ties by slot), padding last."""
    ids_row = np.asarray(ids_row, np.int64)
    K = ids_row.shape[0]
    slots = np.arange(K)
    valid = ids_row >= 0
    key = np.where(valid, ids_row, np.iinfo(np.int64).max)
    return np.lexsort((slots, key))  # primary key: id (padding last), then slot


def canonicalize(ids, logits):
    """ids int32 [Q, K], logits float32 [Q, K] -> (ids_out, logits_out, probs_out)."""
    ids = np.asarray(ids, np.int32)
    logits = np.asarray(logits, np.float32)
    Q, K = ids.shape
    ids_out = np.empty_like(ids)
    lg_out = np.empty_like(logits)
    probs = np.zeros((Q, K), np.float32)
    for q in range(Q):
        perm = canonical_order(ids[q])
        ids_out[q] = ids[q][perm]
        lg_out[q] = logits[q][perm]
        valid = ids_out[q] >= 0
        nv = int(valid.sum())
        if nv == 0:
            continue
        lv = lg_out[q][:nv]  # valid slots come first
        m = np.max(lv)
        e = detmath.exp32((lv - m).astype(np.float32))
        S = np.float32(-0.0)
        for x in e:
            S = np.float32(S + x)
        probs[q, :nv] = (e / S).astype(np.float32)
    return ids_out, lg_out, probs
