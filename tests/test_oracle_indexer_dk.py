"""Pins of the fused indexer-dK oracle (oracle/indexer_dk.py).

  * the float64 gradient of the clipped KL loss by central differences (signs,
    the row sum, which query row a slot takes, duplicate ids in a row);
  * exact dyadic inputs, where every step is exact and the result is the exact
    sum;
  * a scalar brute-force restatement (oracle/brute.py) on tiny inputs with
    padding, out-of-range ids, zero, negative-zero and subnormal targets;
  * the clamp: targets below the float32 nearest e^-100 become that value on
    valid slots; dropped slots change neither the row sum nor dK.
"""
import math

import numpy as np
import pytest

import workloads as W
from oracle import brute, index_add as oi, indexer_dk as ok
from oracle.primitives import widen_bf16


def bits(x):
    return np.asarray(x, np.float32).view(np.uint32)


def test_eps_is_the_float32_nearest_e_minus_100():
    assert ok.eps() == np.float32(math.exp(-100.0))
    assert ok.eps().view(np.uint32) == 27
    assert abs(27 * 2.0 ** -149 - math.exp(-100)) < abs(26 * 2.0 ** -149 - math.exp(-100))


def test_clamp_and_dropped_slots():
    ids = np.array([[3, -1, 7, 2, 9]], np.int32)   # n_rows 8: 9 is out of range, -1 padding
    t = np.array([[0.0, 0.4, -0.0, 1e-45, 0.25]], np.float32)
    kept = ok.kept_targets(ids, t, 8)
    assert bits(kept).tolist() == [[27, 0, 27, 27, 0]]
    kept2 = ok.kept_targets(np.array([[1]], np.int32), np.array([[0.125]], np.float32), 8)
    assert kept2[0, 0] == np.float32(0.125)
    # dropped slots: whatever their predict/target, coefficients and the row sum ignore them
    p = np.array([[0.5, 0.9, 0.25, 0.125, 0.7]], np.float32)
    c = ok.coefficients(ids, p, t, 8, 1.0)
    assert c[0, 1] == 0 and c[0, 4] == 0
    S = ok.row_sums(kept)[0]
    assert S.view(np.uint32) == 81   # three clamped slots, 27 * 2^-149 each, exactly
    # 0.5 * S = 40.5 units rounds to the even 40, minus 27 leaves 13 units of 2^-149
    assert c[0, 0].view(np.uint32) == 13


def test_exact_dyadic_inputs_give_the_exact_sum():
    inp = W.indexer_dk_inputs(Q=64, K=16, n_rows=40, dim=8, seed=3, integer=True)
    got = ok.indexer_dk(inp.dk0, inp.ids, inp.predict, inp.target, inp.q, inp.scale, 5)
    valid = (inp.ids >= 0) & (inp.ids < 40)
    kept = np.where(valid, inp.target.astype(np.float64), 0.0)
    S = kept.sum(1)
    c = np.where(valid, (inp.predict * S[:, None] - kept) * float(inp.scale), 0.0)
    q = widen_bf16(inp.q).astype(np.float64)
    exact = inp.dk0.astype(np.float64).copy()
    for r in range(64):
        for j in range(16):
            if valid[r, j]:
                exact[inp.ids[r, j]] += c[r, j] * q[r]
    assert np.all(np.abs(exact) * 512 < 2 ** 24)   # every partial sum is an exact float32
    assert np.array_equal(got.astype(np.float64), exact)


def test_central_difference_of_the_clipped_kl_loss():
    rng = np.random.default_rng(5)
    Q, K, n_rows, D = 3, 7, 5, 4
    ids = np.array([[0, 2, 2, -1, 4, 1, 3], [4, 4, 0, 1, -1, -1, 2], [3, 1, 0, 2, 4, 0, 1]], np.int32)
    q = W.bf16_bits(rng.standard_normal((Q, D)).astype(np.float32))
    qf = widen_bf16(q).astype(np.float64)
    Kmat = rng.standard_normal((n_rows, D))
    sm, scale0 = 0.5, 0.03
    target = rng.random((Q, K)).astype(np.float32)
    target[1, 3] = 0.0  # below e^-100 on a valid slot: clamped
    valid = ids >= 0
    kept = np.where(valid, np.maximum(target.astype(np.float64), float(ok.eps())), 0.0)

    def probs(Km):
        s = np.where(valid, sm * np.einsum("rd,rjd->rj", qf, Km[np.where(valid, ids, 0)]), -np.inf)
        e = np.where(valid, np.exp(s - s.max(1, keepdims=True)), 0.0)
        return e / e.sum(1, keepdims=True)

    def loss(Km):
        p = probs(Km)
        return scale0 * np.sum(np.where(valid, kept * (np.log(np.where(valid, kept, 1.0)) - np.log(np.where(valid, p, 1.0))), 0.0))

    fd = np.zeros_like(Kmat)
    h = 1e-6
    for m in range(n_rows):
        for d in range(D):
            Kp, Km = Kmat.copy(), Kmat.copy()
            Kp[m, d] += h; Km[m, d] -= h
            fd[m, d] = (loss(Kp) - loss(Km)) / (2 * h)
    predict = probs(Kmat).astype(np.float32)
    got = ok.indexer_dk(np.zeros((n_rows, D), np.float32), ids, predict, target, q, np.float32(scale0 * sm), 2)
    err = np.linalg.norm(got - fd) / np.linalg.norm(fd)
    assert err < 1e-5, err


@pytest.mark.parametrize("L", [1, 3, 1000])
def test_brute_force_tiny(L):
    rng = np.random.default_rng(L)
    Q, K, n_rows, D = 5, 9, 6, 3
    ids = rng.integers(-1, n_rows, (Q, K)).astype(np.int32)
    ids[0, 2] = 6      # out of range: dropped
    ids[1, :] = -1     # an all-padding row
    ids[2, 4] = -7
    predict = rng.random((Q, K)).astype(np.float32)
    target = rng.random((Q, K)).astype(np.float32)
    target[3, 1], target[3, 2], target[4, 0] = 0.0, -0.0, 1e-45
    q = W.bf16_bits(rng.standard_normal((Q, D)).astype(np.float32))
    dk0 = rng.standard_normal((n_rows, D)).astype(np.float32)
    scale = np.float32(0.0123)
    got = ok.indexer_dk(dk0, ids, predict, target, q, scale, L)
    want = brute.indexer_dk(dk0, ids, predict, target, q, scale, L)
    assert np.array_equal(bits(got), bits(want))


def test_power_of_two_scaling_and_composition():
    inp = W.indexer_dk_inputs(Q=32, K=24, n_rows=50, dim=8, seed=9)
    a = ok.indexer_dk(np.zeros((50, 8), np.float32), inp.ids, inp.predict, inp.target, inp.q, inp.scale, 4)
    b = ok.indexer_dk(np.zeros((50, 8), np.float32), inp.ids, inp.predict, inp.target, inp.q,
                      np.float32(inp.scale * 4), 4)
    assert np.array_equal(bits(b), bits(a * np.float32(4)))
    # the fused accumulation is the canonical index_add of the explicit float32 source rows
    coef = ok.coefficients(inp.ids, inp.predict, inp.target, 50, inp.scale)
    src = ok.source_rows(coef, inp.q)
    c = oi.index_add(inp.dk0, inp.ids.reshape(-1), src, 4)
    assert np.array_equal(bits(c), bits(ok.indexer_dk(inp.dk0, inp.ids, inp.predict, inp.target, inp.q,
                                                        inp.scale, 4)))
