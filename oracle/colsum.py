"""Gate-backward column sums, ordered (test infrastructure only).

Megatron-LM PR #8244 (ordered A_log/dt_bias reduction in the fused pre-GDR
gate backward), description: in deterministic mode the per-program FP32
partials are kept apart and summed afterwards, in a fixed order, on the stream
the backward runs on; a rule on the shape alone picks the tile, which also
fixes the scratch size.
The page names only the two gradients; the gate itself is the Gated-DeltaNet
one, g = -exp(A_log[h]) * softplus(a[t,h] + dt_bias[h]), whose parameter
gradients are

    dA_log[h]   = sum_t dg[t,h] * g[t,h]
    ddt_bias[h] = sum_t dg[t,h] * (-exp(A_log[h])) * sigmoid(a[t,h] + dt_bias[h]).

Canonical order for a tile of BT rows (BT a power of two): the adjacent
pairwise tree over the tile's rows (rows past T are -0.0), one slot per
(tile, head); then the slots of each head are folded left to right in tile
order and the total is added once into the output. The head-block size BH of
the launch does not enter the arithmetic.

Per-element operation order (binary32, no fused multiply-add):
    x  = f32(a) + dt_bias[h];  nA = -exp32(A_log[h]);  e = exp32(-|x|)
    sp = softplus32(x);        sg = sigmoid32(x)      (both from the same e)
    t1 = f32(dg) * (nA * sp);  t2 = f32(dg) * (nA * sg)

The elementwise gradient of the gate input (the scope table's gate-variants
row; the page itself names only the two parameter gradients): x depends on
a[t,h] and dt_bias[h] alike, so da[t,h] = dg * dg/da is the same term t2,
kept per element and stored in the input precision (bf16 round to nearest
even for bf16 inputs, float32 as is).
"""
from __future__ import annotations

import numpy as np

from . import detmath
from .primitives import accumulate, narrow_bf16, pairwise, sequential, tiles, widen_bf16


def gate_input(x) -> np.ndarray:
    """Gate inputs arrive as bf16 bit patterns (uint16, widened exactly) or as
    float32 values (the GDN gate page tests both input precisions)."""
    x = np.asarray(x)
    return x.astype(np.float32) if x.dtype == np.float32 else widen_bf16(x)


def gate_terms(a_bits, dg_bits, A_log, dt_bias):
    """Elementwise terms (t1, t2), each [T, H] float32."""
    a = gate_input(a_bits)
    dg = gate_input(dg_bits)
    A_log = np.asarray(A_log, np.float32)
    dt_bias = np.asarray(dt_bias, np.float32)
    x = (a + dt_bias[None, :]).astype(np.float32)
    nA = -detmath.exp32(A_log)
    e = detmath.exp32(-np.abs(x))
    sp = detmath.softplus_from(x, e)
    sg = detmath.sigmoid_from(x, e)
    g = nA[None, :] * sp
    t1 = dg * g
    t2 = dg * (nA[None, :] * sg)
    return t1.astype(np.float32), t2.astype(np.float32)


def gate_da(a_bits, dg_bits, A_log, dt_bias) -> np.ndarray:
    """da [T, H]: t2 per element, as bf16 bits (uint16) for bf16 inputs and
    float32 for float32 inputs."""
    _, t2 = gate_terms(a_bits, dg_bits, A_log, dt_bias)
    return t2 if np.asarray(a_bits).dtype == np.float32 else narrow_bf16(t2)


def gate_slots(a_bits, dg_bits, A_log, dt_bias, block_t: int):
    """Per-tile partials (slot1, slot2), each [ceil(T/BT), H]."""
    t1, t2 = gate_terms(a_bits, dg_bits, A_log, dt_bias)
    return pairwise(tiles(t1, block_t, axis=0)), pairwise(tiles(t2, block_t, axis=0))


def colsum(a_bits, dg_bits, A_log, dt_bias, dA_log0, ddt_bias0, block_t: int):
    """Return (dA_log, ddt_bias) after accumulating the ordered column sums."""
    s1, s2 = gate_slots(a_bits, dg_bits, A_log, dt_bias, block_t)
    return accumulate(dA_log0, sequential(s1, axis=0)), accumulate(ddt_bias0, sequential(s2, axis=0))
