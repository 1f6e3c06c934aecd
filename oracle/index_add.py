"""Deterministic index_add for the sparse-indexer dK (test infrastructure only).

Megatron-LM PR #7441 (DSv4 deterministic mode), source 3: the indexer backward
accumulated dK with atomics; the fix computes it without atomics through a
deterministic index_add whose fallback sorts the ids stably and takes a prefix
sum of the counts, and padding slots are dropped.

    out[id] += src[p]   for every source row p with ids[p] = id >= 0

Canonical order (the reading taken here):
1. keep the pairs (ids[p], p) with 0 <= ids[p] < n_rows; ids of -1 are
   padding and any other out-of-range id is dropped as well;
2. sort the pairs by id, stably, so rows with equal ids stay in ascending p
   (the prefix sum of the sort is the integer exclusive scan of key counts,
   which gives each id's segment of the sorted list);
3. cut each id's run r_0 .. r_{n-1} into chunks of L consecutive rows;
   each chunk's partial is the left-to-right fold of its rows, per dim;
4. fold the chunk partials of an id left to right and add the total once
   into out[id]. Ids with no rows are untouched.

With L at least the longest run this is exactly the literal sequential loop
that adds the source rows of each id into out[id] one by one, in stable id
order, when out starts at +0.
"""
from __future__ import annotations

import numpy as np

from .primitives import NEG_ZERO, accumulate, widen_bf16


def stable_order(ids, n_rows: int):
    """Return (perm, counts): source rows in stable id order and per-id counts."""
    ids = np.asarray(ids, np.int64)
    valid = np.nonzero((ids >= 0) & (ids < n_rows))[0]
    keys = ids[valid]
    order = np.argsort(keys, kind="stable")
    perm = valid[order]
    counts = np.bincount(keys, minlength=n_rows)
    return perm.astype(np.int64), counts.astype(np.int64)


def chunk_partials(src_f32: np.ndarray, perm: np.ndarray, counts: np.ndarray, L: int):
    """Return (chunk_key, chunk_part): one row of partial sums per chunk, in key order."""
    seg_off = np.concatenate([[0], np.cumsum(counts)])
    n_chunks = -(-counts // L)
    keys = np.repeat(np.arange(len(counts)), n_chunks)
    j = np.arange(len(keys)) - np.repeat(np.concatenate([[0], np.cumsum(n_chunks)])[:-1], n_chunks)
    start = seg_off[keys] + j * L
    length = np.minimum(L, seg_off[keys + 1] - start)
    D = src_f32.shape[1]
    part = np.full((len(keys), D), NEG_ZERO, np.float32)
    for i in range(int(length.max()) if len(length) else 0):
        m = np.nonzero(length > i)[0]
        part[m] = np.add(part[m], src_f32[perm[start[m] + i]], dtype=np.float32)
    return keys, part, n_chunks


def index_add(out0, ids, src_bits, chunk_rows: int):
    """Return out0 with the canonical index_add applied (out0 is not modified)."""
    out = np.array(out0, np.float32, copy=True)
    n_rows, D = out.shape
    perm, counts = stable_order(ids, n_rows)
    if len(perm) == 0:
        return out
    src = np.asarray(src_bits)
    src = src.astype(np.float32) if src.dtype == np.float32 else widen_bf16(src)  # float32 values or bf16 bits
    keys, part, n_chunks = chunk_partials(src, perm, counts, chunk_rows)
    first = np.concatenate([[0], np.cumsum(n_chunks)])
    present = np.nonzero(counts)[0]
    total = np.full((len(present), D), NEG_ZERO, np.float32)
    for j in range(int(n_chunks.max())):
        m = np.nonzero(n_chunks[present] > j)[0]
        total[m] = np.add(total[m], part[first[present[m]] + j], dtype=np.float32)
    out[present] = accumulate(out[present], total)
    return out
