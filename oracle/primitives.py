"""Reduction primitives shared by the four oracle cases (test infrastructure only).

The pages fix the pattern but not the in-tile order: each program/CTA writes
its own FP32 partial into a slot, and the slots are then reduced in a fixed
order on the caller's stream (Megatron-LM PR #8244, description; cudnn-frontend
PR #521, first commit: one slot per subtile, folded by the wrapper in a fixed
order). The readings taken here:

* inside a tile: the adjacent pairwise tree. Level one adds elements (2i, 2i+1),
  the next level adds neighbouring results, and so on to a single value;
  positions past the end of the data are -0.0;
* across slots: a strict left-to-right fold starting from -0.0;
* into the output: one add of the finished total, out <- RN32(out + total),
  i.e. accumulate rather than overwrite (cudnn-frontend PR #521: the slot
  reduction adds into the existing output; FlashInfer PR #8924: the result
  equals AccumulateGrad of the deterministic dW).

-0.0 is the exact additive identity of binary32 (x + -0.0 == x for every x,
including -0.0), so padding never changes a bit and an empty set leaves the
output bitwise unchanged (FlashInfer PR #8602, commits: its tests require an
empty group to leave the output bit-identical).
"""
from __future__ import annotations

import numpy as np

F32 = np.float32
NEG_ZERO = np.float32(-0.0)


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """Exact bfloat16 -> float32 widening of raw uint16 bit patterns."""
    return (np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def narrow_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest, ties to
    the even significand; NaN stays NaN (quiet), infinities and signed zeros
    are kept. Written on the bit pattern: adding 0x7FFF plus the lowest kept
    bit carries into the kept part exactly when the dropped half-word is above
    the midpoint, or at it with an odd kept part."""
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    r = np.where(nan, (u >> 16) | 0x0040, r)
    return (r & 0xFFFF).astype(np.uint16)


def tiles(x: np.ndarray, block: int, axis: int) -> np.ndarray:
    """Split ``axis`` into consecutive tiles of ``block`` elements.

    The last tile is padded with -0.0. The tile index becomes ``axis`` and the
    position inside the tile becomes a new trailing axis.
    """
    x = np.moveaxis(np.asarray(x, np.float32), axis, -1)
    n = x.shape[-1]
    n_tiles = -(-n // block)
    pad = n_tiles * block - n
    if pad:
        x = np.concatenate([x, np.full(x.shape[:-1] + (pad,), NEG_ZERO, np.float32)], axis=-1)
    x = x.reshape(x.shape[:-1] + (n_tiles, block))
    return np.moveaxis(x, -2, axis if axis >= 0 else axis - 1)


def pairwise(x: np.ndarray) -> np.ndarray:
    """Adjacent pairwise tree over the last axis (its length must be a power of two)."""
    x = np.asarray(x, np.float32)
    n = x.shape[-1]
    if n <= 0 or n & (n - 1):
        raise ValueError("pairwise tree needs a power-of-two length, got %d" % n)
    while x.shape[-1] > 1:
        x = np.add(x[..., 0::2], x[..., 1::2], dtype=np.float32)
    return x[..., 0]


def sequential(x: np.ndarray, axis: int = -1) -> np.ndarray:
    """Left-to-right fold ((x0 + x1) + x2) + ... along ``axis``; an empty fold is -0.0."""
    x = np.moveaxis(np.asarray(x, np.float32), axis, 0)
    acc = np.full(x.shape[1:], NEG_ZERO, np.float32)
    for i in range(x.shape[0]):
        acc = np.add(acc, x[i], dtype=np.float32)
    return acc


def accumulate(out: np.ndarray, total: np.ndarray) -> np.ndarray:
    """out <- RN32(out + total), one rounding."""
    return np.add(np.asarray(out, np.float32), np.asarray(total, np.float32), dtype=np.float32)
