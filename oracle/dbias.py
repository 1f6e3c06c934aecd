"""Grouped dsReLU backward dbias with per-M-tile slots (test infrastructure only).

cudnn-frontend PR #521 (deterministic dprob/dbias in the grouped-GEMM dsReLU
backward), the commit that extends the determinism flag to dbias: dbias is a
column sum over tokens, so its contention is across M tiles (dprob's is across
N tiles). It gets its own float32 workspace with one slot per absolute M block
and column, and a per-expert segment sum of the slots; the kernel's check
requires every expert to start on an M-tile boundary, so no tile holds rows of
two experts.

    dbias[e, n] += sum_{m in expert e} dA[m, n]

Canonical order (the reading taken here):
* expert boundaries from device offsets, clamped monotone:
  b_0 = clamp(offs[0], 0, M), b_e = clamp(offs[e], b_{e-1}, M);
* expert e's rows [b_e, b_{e+1}) are cut into tiles of ``block_m`` rows counted
  from b_e (when every b_e is a multiple of block_m these are exactly the
  page's absolute M blocks; unaligned experts are allowed here and never share
  a tile); rows past b_{e+1} are -0.0;
* slot[t, n] = the adjacent pairwise tree of the tile's block_m values of
  column n;
* dbias[e, n] <- RN32(dbias[e, n] + fold(slots of e's tiles in tile order)),
  fold the left-to-right sum from -0.0. An expert with no rows leaves its row
  bitwise unchanged.
The slots stay float32 (a later commit on the page narrows them to bf16 to
match its bf16 dbias output; here the output is float32 and accumulated).
"""
from __future__ import annotations

import numpy as np

from .primitives import accumulate, pairwise, sequential, tiles, widen_bf16

BLOCK_M = 128


def expert_bounds(offs, M: int):
    """Clamped monotone expert boundaries b_0 .. b_E."""
    b = []
    prev = 0
    for e, o in enumerate(np.asarray(offs, np.int64)):
        lo = 0 if e == 0 else prev
        v = int(min(max(int(o), lo), M))
        b.append(v)
        prev = v
    return b


def tile_ranges(offs, M: int, block_m: int = BLOCK_M):
    """Per expert, the (row_begin, row_end) of its tiles in order."""
    b = expert_bounds(offs, M)
    return [[(r, min(r + block_m, b[e + 1])) for r in range(b[e], b[e + 1], block_m)] for e in range(len(b) - 1)]


def expert_slots(dA_bits, r0: int, r1: int, block_m: int = BLOCK_M) -> np.ndarray:
    """[n_tiles, N] slots of the rows [r0, r1) of one expert."""
    x = widen_bf16(dA_bits[r0:r1])
    return pairwise(tiles(x, block_m, axis=0))


def grouped_dbias(dbias0, dA_bits, offs, block_m: int = BLOCK_M) -> np.ndarray:
    dbias0 = np.asarray(dbias0, np.float32)
    M = dA_bits.shape[0]
    b = expert_bounds(offs, M)
    out = dbias0.copy()
    for e in range(len(b) - 1):
        if b[e + 1] > b[e]:
            total = sequential(expert_slots(dA_bits, b[e], b[e + 1], block_m), axis=0)
            out[e] = accumulate(out[e], total)
    return out
