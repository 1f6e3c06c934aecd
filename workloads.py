"""Seeded synthetic inputs for the four deterministic gradient reductions.

This module only draws random inputs and rounds them to bfloat16 storage. It
holds none of the reductions' arithmetic, so both the CPU oracle and the GPU
library can be fed from it without sharing any compute code.

Every tensor comes from ``numpy.random.default_rng([seed, tensor_id])`` so a
given (seed, shape) always produces the same bits on any host. bfloat16 values
are returned as their raw ``uint16`` bit patterns (round-to-nearest-even from
float32), which is how they are uploaded to the device.

Workload shapes follow the pages' four cases (Megatron-LM PR #8244 gate
backward; Megatron-LM PR #7441 indexer dK; cudnn-frontend PR #521 grouped-GEMM
dprob; FlashInfer PR #8602/#8924 grouped weight-gradient accumulate).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "bf16_bits", "GateInputs", "gate_inputs", "IndexAddInputs", "index_add_inputs",
    "DprobInputs", "dprob_inputs", "WgradInputs", "wgrad_inputs",
]


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    # finite inputs never carry out of 32 bits: the largest is 0xFF7FFFFF + 0x8000
    r = (u >> np.uint32(16)) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= np.uint32(16)
    return r.astype(np.uint16)


def _rng(seed: int, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng([seed, tensor_id])


# --------------------------------------------------------------------------- gate
@dataclass
class GateInputs:
    """Gated-DeltaNet gate backward inputs.

    ``a`` is a contiguous [T, H] bf16 tensor. ``dg_base`` is a [T, 2H] bf16
    tensor whose columns H..2H-1 form the strided ``dg`` view (row stride 2H,
    element offset H), matching the non-contiguous gradient the pages test.
    """
    T: int
    H: int
    a: np.ndarray          # uint16 [T, H] bf16 bits (or float32 values)
    dg_base: np.ndarray    # uint16 [T, 2H] bf16 bits (or float32 values)
    A_log: np.ndarray      # float32 [H]
    dt_bias: np.ndarray    # float32 [H]
    dA_log0: np.ndarray    # float32 [H] initial accumulator
    ddt_bias0: np.ndarray  # float32 [H]

    @property
    def dg(self) -> np.ndarray:
        return self.dg_base[:, self.H:]


def gate_inputs(T: int, H: int, seed: int = 1, out_init: str = "zero", dtype: str = "bf16") -> GateInputs:
    """``dtype="f32"`` keeps ``a`` and ``dg_base`` as float32 values (the same
    draws, not rounded to bf16) instead of bf16 bit patterns."""
    a = _rng(seed, 0).standard_normal((T, H), dtype=np.float32)
    dg_base = _rng(seed, 1).standard_normal((T, 2 * H), dtype=np.float32)
    if dtype == "bf16":
        a, dg_base = bf16_bits(a), bf16_bits(dg_base)
    elif dtype != "f32":
        raise ValueError("dtype must be bf16 or f32")
    A_log = _rng(seed, 2).uniform(-2.0, 1.0, H).astype(np.float32)
    dt_bias = _rng(seed, 3).uniform(-1.0, 1.0, H).astype(np.float32)
    if out_init == "zero":
        o1 = np.zeros(H, np.float32); o2 = np.zeros(H, np.float32)
    else:
        o1 = _rng(seed, 4).standard_normal(H, dtype=np.float32)
        o2 = _rng(seed, 5).standard_normal(H, dtype=np.float32)
    return GateInputs(T, H, a, dg_base, A_log, dt_bias, o1, o2)


# ---------------------------------------------------------------------- index_add
@dataclass
class IndexAddInputs:
    """Sparse-indexer dK scatter: ``out[ids[p]] += src[p]`` for ids >= 0.

    ``ids`` is the flattened [Q, K] top-k id matrix (int32, -1 = padding),
    ``src`` the [Q*K, D] bf16 rows, ``out0`` the [n_rows, D] float32 start.
    """
    n_rows: int
    dim: int
    ids: np.ndarray   # int32 [P]
    src: np.ndarray   # uint16 [P, D] bf16 bits (or float32 values)
    out0: np.ndarray  # float32 [n_rows, D]


def zipf_ids(P: int, n_rows: int, s: float, pad_frac: float, seed: int, tensor_id: int = 0) -> np.ndarray:
    """i.i.d. Zipf(s) ranks mapped to keys by a seeded permutation; padding -1."""
    rng = _rng(seed, tensor_id)
    w = np.arange(1, n_rows + 1, dtype=np.float64) ** (-s)
    cdf = np.cumsum(w / w.sum())
    cdf[-1] = 1.0
    ranks = np.searchsorted(cdf, rng.random(P), side="right")
    ranks = np.minimum(ranks, n_rows - 1)
    perm = rng.permutation(n_rows).astype(np.int32)
    ids = perm[ranks]
    pad = rng.random(P) < pad_frac
    ids[pad] = -1
    return ids.astype(np.int32)


def index_add_inputs(Q: int = 4096, K: int = 512, n_rows: int = 8192, dim: int = 128, seed: int = 3,
                     zipf_s: float = 1.1, pad_frac: float = 0.05, src_std: float = 0.02,
                     out_init: str = "zero", dtype: str = "bf16") -> IndexAddInputs:
    """``dtype="f32"`` keeps ``src`` as float32 values (the same draws)."""
    P = Q * K
    ids = zipf_ids(P, n_rows, zipf_s, pad_frac, seed, 0)
    src = _rng(seed, 1).standard_normal((P, dim), dtype=np.float32) * np.float32(src_std)
    if dtype == "bf16":
        src = bf16_bits(src)
    elif dtype != "f32":
        raise ValueError("dtype must be bf16 or f32")
    if out_init == "zero":
        out0 = np.zeros((n_rows, dim), np.float32)
    else:
        out0 = _rng(seed, 2).standard_normal((n_rows, dim), dtype=np.float32)
    return IndexAddInputs(n_rows, dim, ids, src, out0)


# --------------------------------------------------------- fused indexer dK source
@dataclass
class IndexerDkInputs:
    """Sparse-indexer dK with its source rows made from the score gradient:
    per query row r and top-k slot j an id (-1 = padding), the indexer's
    softmax ``predict`` over the row's valid slots, the attention ``target``
    (rows summing to 0.5, a few entries below e^-100 or zero), the indexer
    query rows ``q`` and the float32 normalisation ``scale``."""
    n_rows: int
    dim: int
    ids: np.ndarray      # int32 [Q, K]
    predict: np.ndarray  # float32 [Q, K]
    target: np.ndarray   # float32 [Q, K]
    q: np.ndarray        # uint16 [Q, D] bf16 bits
    scale: np.float32
    dk0: np.ndarray      # float32 [n_rows, D]


def indexer_dk_ids(Q: int = 4096, K: int = 512, n_rows: int = 8192, seed: int = 8, zipf_s: float = 1.1,
                   pad_frac: float = 0.05) -> np.ndarray:
    """The [Q, K] key ids of the fused indexer-dK workload (the index_add id recipe, one row per query)."""
    return zipf_ids(Q * K, n_rows, zipf_s, pad_frac, seed, 0).reshape(Q, K)


def indexer_dk_inputs(Q: int = 4096, K: int = 512, n_rows: int = 8192, dim: int = 128, seed: int = 8,
                      zipf_s: float = 1.1, pad_frac: float = 0.05, out_init: str = "zero",
                      loss_coeff: float = 0.1, batch: int = 1, sm_scale=None, grad_loss: float = 1.0,
                      integer: bool = False) -> IndexerDkInputs:
    """Ids as for the index_add workload (Zipf over keys, duplicates, 5% padding); predict = softmax of
    N(0,1) logits over the valid slots (float64, rounded once); target = U(0,1) weights normalised to 0.5
    per row with 2% of slots replaced by 0, -0, subnormals or values below e^-100; q ~ N(0,1) bf16.
    ``integer`` draws small dyadic predict, target and q and a power-of-two scale instead, so that every
    step is exact."""
    ids = indexer_dk_ids(Q, K, n_rows, seed, zipf_s, pad_frac)
    valid = (ids >= 0) & (ids < n_rows)
    rng = _rng(seed, 1)
    if integer:
        predict = (rng.integers(0, 9, (Q, K)) / 8.0).astype(np.float32)
        target = (rng.integers(1, 17, (Q, K)) / 16.0).astype(np.float32)
        q = bf16_bits(rng.integers(-2, 3, (Q, dim)).astype(np.float32))
        scale = np.float32(0.25)
    else:
        lg = rng.standard_normal((Q, K))
        lg = np.where(valid, lg, -np.inf)
        m = np.max(np.where(valid, lg, -1e300), axis=1, keepdims=True)
        e = np.where(valid, np.exp(lg - m), 0.0)
        predict = (e / np.maximum(e.sum(1, keepdims=True), 1e-300)).astype(np.float32)
        w = rng.random((Q, K))
        target = (0.5 * w / w.sum(1, keepdims=True)).astype(np.float32)
        tiny = rng.random((Q, K)) < 0.02
        tiny_vals = np.array([0.0, -0.0, 1e-45, 2.8e-45, 3.0e-44, 4.0e-44, 1e-40, 1e-30], np.float32)
        target[tiny] = tiny_vals[rng.integers(0, len(tiny_vals), int(tiny.sum()))]
        q = bf16_bits(_rng(seed, 2).standard_normal((Q, dim), dtype=np.float32))
        sm = 1.0 / np.sqrt(dim) if sm_scale is None else sm_scale
        scale = np.float32(loss_coeff / (batch * Q) * sm * grad_loss)
    if out_init == "zero":
        dk0 = np.zeros((n_rows, dim), np.float32)
    else:
        dk0 = _rng(seed, 3).standard_normal((n_rows, dim), dtype=np.float32)
    return IndexerDkInputs(n_rows, dim, ids.astype(np.int32), predict, target, q, scale, dk0)


# -------------------------------------------------------------------------- dprob
@dataclass
class DprobInputs:
    """Grouped-GEMM dsReLU backward dprob inputs (rows grouped by expert)."""
    M: int
    N: int
    offs: np.ndarray   # int32 [E+1] expert row offsets
    dY: np.ndarray     # uint16 [M, N]
    C: np.ndarray      # uint16 [M, N]
    dprob0: np.ndarray  # float32 [M]


def expert_counts(total: int, E: int, min_tokens: int, seed: int, tensor_id: int = 0) -> np.ndarray:
    rng = _rng(seed, tensor_id)
    extra = rng.multinomial(total - E * min_tokens, [1.0 / E] * E)
    return (min_tokens + extra).astype(np.int64)


def dprob_inputs(M: int = 16384, N: int = 2048, E: int = 8, min_tokens: int = 256, seed: int = 4,
                 out_init: str = "zero") -> DprobInputs:
    counts = expert_counts(M, E, min_tokens, seed, 0) if M >= E * min_tokens else \
        np.array([M // E + (1 if e < M % E else 0) for e in range(E)], np.int64)
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    dY = bf16_bits(_rng(seed, 1).standard_normal((M, N), dtype=np.float32))
    C = bf16_bits(_rng(seed, 2).standard_normal((M, N), dtype=np.float32))
    if out_init == "zero":
        d0 = np.zeros(M, np.float32)
    else:
        d0 = _rng(seed, 3).standard_normal(M, dtype=np.float32)
    return DprobInputs(M, N, offs, dY, C, d0)


# -------------------------------------------------------------------------- dbias
@dataclass
class DbiasInputs:
    """Grouped dsReLU backward dbias inputs: per-expert column sums of dA."""
    M: int
    N: int
    offs: np.ndarray    # int32 [E+1] expert row offsets
    dA: np.ndarray      # uint16 [M, N]
    dbias0: np.ndarray  # float32 [E, N]


def dbias_inputs(M: int = 16384, N: int = 2048, E: int = 8, min_tokens: int = 256, seed: int = 6,
                 out_init: str = "zero", integer: bool = False) -> DbiasInputs:
    """Expert sizes as for dprob (min_tokens + a uniform multinomial); dA ~ N(0, 1)
    (or small integers in [-4, 4]); dbias0 zero or N(0, 1)."""
    counts = expert_counts(M, E, min_tokens, seed, 0) if M >= E * min_tokens else \
        np.array([M // E + (1 if e < M % E else 0) for e in range(E)], np.int64)
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    if integer:
        dA = bf16_bits(_rng(seed, 1).integers(-4, 5, size=(M, N)).astype(np.float32))
    else:
        dA = bf16_bits(_rng(seed, 1).standard_normal((M, N), dtype=np.float32))
    if out_init == "zero":
        d0 = np.zeros((E, N), np.float32)
    else:
        d0 = _rng(seed, 2).standard_normal((E, N), dtype=np.float32)
    return DbiasInputs(M, N, offs, dA, d0)


# ------------------------------------------------------------- compact top-k
@dataclass
class TopkInputs:
    """Compact indexer top-k rows: ids (distinct per row, in a shuffled slot order,
    -1 padding) and their logits."""
    ids: np.ndarray     # int32 [Q, K]
    logits: np.ndarray  # float32 [Q, K]


def topk_inputs(Q: int = 4096, K: int = 512, n_keys: int = 8192, pad_frac: float = 0.05, seed: int = 7,
                distinct: bool = True) -> TopkInputs:
    """Per row: K keys drawn without replacement (with replacement when
    ``distinct`` is False), i.i.d. padding slots, logits ~ N(0, 1); the slot
    order is a random shuffle, as a run-dependent selection order would be."""
    rng = _rng(seed, 0)
    if distinct:
        ids = np.argsort(rng.random((Q, n_keys)), axis=1)[:, :K].astype(np.int32)
    else:
        ids = rng.integers(0, n_keys, size=(Q, K)).astype(np.int32)
    pad = _rng(seed, 1).random((Q, K)) < pad_frac
    ids = np.where(pad, np.int32(-1), ids)
    logits = _rng(seed, 2).standard_normal((Q, K), dtype=np.float32)
    return TopkInputs(ids, logits)


# -------------------------------------------------------------------------- wgrad
@dataclass
class WgradInputs:
    """Grouped weight gradient: main_grad[e] += G_e^T X_e over expert row ranges."""
    M: int
    N: int
    offs: np.ndarray       # int32 [E+1]
    G: np.ndarray          # uint16 [T_total, M]
    X: np.ndarray          # uint16 [T_total, N]
    main_grad0: np.ndarray  # float32 [E, M, N]
    tokens: np.ndarray = field(default=None)


def wgrad_tokens(E: int = 8, t_lo: int = 1024, t_hi: int = 8192, seed: int = 5) -> np.ndarray:
    """Token rows per expert of the grouped weight-gradient workload, U{t_lo..t_hi}."""
    return _rng(seed, 0).integers(t_lo, t_hi + 1, size=E)


def wgrad_inputs(E: int = 8, M: int = 1408, N: int = 2048, tokens=None, t_lo: int = 1024, t_hi: int = 8192,
                 seed: int = 5, std: float = 0.02, out_init: str = "zero", integer: bool = False) -> WgradInputs:
    if tokens is None:
        tokens = wgrad_tokens(E, t_lo, t_hi, seed)
    tokens = np.asarray(tokens, np.int64)
    offs = np.concatenate([[0], np.cumsum(tokens)]).astype(np.int32)
    T = int(offs[-1])
    if integer:
        G = bf16_bits(_rng(seed, 1).integers(-2, 3, size=(T, M)).astype(np.float32))
        X = bf16_bits(_rng(seed, 2).integers(-2, 3, size=(T, N)).astype(np.float32))
    else:
        G = bf16_bits(_rng(seed, 1).standard_normal((T, M), dtype=np.float32) * np.float32(std))
        X = bf16_bits(_rng(seed, 2).standard_normal((T, N), dtype=np.float32) * np.float32(std))
    if out_init == "zero":
        mg = np.zeros((E, M, N), np.float32)
    elif integer:
        mg = _rng(seed, 3).integers(-8, 9, size=(E, M, N)).astype(np.float32)
    else:
        mg = _rng(seed, 3).standard_normal((E, M, N), dtype=np.float32) * np.float32(1e-2)
    return WgradInputs(M, N, offs, G, X, mg, tokens)
