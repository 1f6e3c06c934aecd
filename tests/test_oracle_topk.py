"""Pins of the canonical compact top-k oracle (CPU): brute force, slot-order
invariance, the float64 softmax bound and the padding rules."""
import numpy as np
import pytest

import workloads as W
from oracle import brute, topk as ot

U = 2.0 ** -24


def bits(x):
    return np.asarray(x, np.float32).view(np.uint32)


@pytest.mark.parametrize("Q,K,n_keys,distinct", [(5, 40, 60, False), (4, 33, 1000, True), (3, 8, 4, False)])
def test_brute_force(Q, K, n_keys, distinct):
    inp = W.topk_inputs(Q=Q, K=K, n_keys=n_keys, seed=K, distinct=distinct, pad_frac=0.2)
    ids, lg = inp.ids.copy(), inp.logits.copy()
    ids[0, :] = -1          # a row that is all padding
    ids[-1, :] = np.abs(ids[-1, :])  # a row without padding
    a = ot.canonicalize(ids, lg)
    b = brute.topk_canonical(ids, lg)
    for x, y in zip(a, b):
        assert np.array_equal(bits(x), bits(y))


def test_slot_order_never_changes_a_bit():
    """The defining property: rows with distinct ids give the same bits whatever
    order the slots arrive in."""
    inp = W.topk_inputs(Q=64, K=512, seed=11)
    ref = ot.canonicalize(inp.ids, inp.logits)
    rng = np.random.default_rng(0)
    for _ in range(3):
        perm = np.argsort(rng.random(inp.ids.shape), axis=1)
        got = ot.canonicalize(np.take_along_axis(inp.ids, perm, 1), np.take_along_axis(inp.logits, perm, 1))
        valid = ref[0] >= 0
        assert np.array_equal(got[0], ref[0])
        assert np.array_equal(bits(got[2]), bits(ref[2]))
        # logits of valid slots; padding slots carry their logits in slot order
        assert np.array_equal(bits(got[1])[valid], bits(ref[1])[valid])


def test_order_padding_and_pairs():
    inp = W.topk_inputs(Q=50, K=100, n_keys=300, seed=12, distinct=False, pad_frac=0.3)
    io, lo, po = ot.canonicalize(inp.ids, inp.logits)
    for q in range(50):
        nv = int((inp.ids[q] >= 0).sum())
        assert np.all(io[q, :nv] >= 0) and np.all(io[q, nv:] < 0)
        assert np.all(np.diff(io[q, :nv]) >= 0)
        # the (id, logit) pairs are a permutation of the input pairs
        a = sorted(zip(inp.ids[q].tolist(), inp.logits[q].view(np.uint32).tolist()))
        b = sorted(zip(io[q].tolist(), lo[q].view(np.uint32).tolist()))
        assert a == b
        assert np.all(po[q, nv:] == 0) and not np.any(np.signbit(po[q, nv:]))


def test_softmax_fp64_bound_and_all_padding_rows():
    inp = W.topk_inputs(Q=40, K=512, seed=13)
    ids = inp.ids.copy(); ids[5] = -1
    io, lo, po = ot.canonicalize(ids, inp.logits)
    for q in range(40):
        nv = int((io[q] >= 0).sum())
        if nv == 0:
            assert np.all(po[q] == 0) and np.all(np.isfinite(po[q]))
            continue
        x = lo[q, :nv].astype(np.float64)
        p64 = np.exp(x - x.max()); p64 /= p64.sum()
        bound = (8 + nv) * U * p64 + 2.0 ** -140
        assert np.all(np.abs(po[q, :nv] - p64) <= bound)
        assert abs(float(po[q, :nv].astype(np.float64).sum()) - 1.0) <= (8 + 2 * nv) * U
