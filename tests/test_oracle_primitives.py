"""Pins of the reduction primitives against closed forms (CPU).

The order-revealing probes follow the FPRev idea: put +M and -M (M = 2^40, so
M absorbs any sum of ones) at two leaves and 1.0 everywhere else. The result
counts the ones that are added after +M and -M have cancelled, which depends
only on the shape of the summation tree:
* adjacent pairwise tree of n leaves: n - size of the smallest aligned block
  holding both leaves = n - 2^bitlength(p XOR q);
* left-to-right fold: the ones after the later of the two positions.
"""
import numpy as np
import pytest

from oracle.primitives import NEG_ZERO, accumulate, pairwise, sequential, tiles, widen_bf16

M = np.float32(2.0 ** 40)


@pytest.mark.parametrize("n", [2, 8, 64, 128, 256])
def test_pairwise_tree_shape(n):
    rng = np.random.default_rng(0)
    pairs = [(p, q) for p in range(n) for q in range(p + 1, n)]
    if len(pairs) > 400:
        pairs = [pairs[i] for i in rng.choice(len(pairs), 400, replace=False)]
    for p, q in pairs:
        x = np.ones(n, np.float32)
        x[p], x[q] = M, -M
        expect = n - 2 ** int(p ^ q).bit_length()
        assert pairwise(x) == expect, (p, q)
        x[p], x[q] = -M, M
        assert pairwise(x) == expect


@pytest.mark.parametrize("n", [1, 2, 5, 16, 33])
def test_sequential_fold_shape(n):
    for p in range(n):
        for q in range(p + 1, n):
            x = np.ones(n, np.float32)
            x[p], x[q] = M, -M
            assert sequential(x) == n - 1 - q


def test_identity_is_negative_zero():
    e = sequential(np.zeros((0,), np.float32))
    assert np.signbit(e) and e == 0
    for v in (np.float32(0.0), np.float32(-0.0), np.float32(1.5), np.float32(-3e-45)):
        s = np.add(v, NEG_ZERO, dtype=np.float32)
        assert s.view(np.uint32) == np.float32(v).view(np.uint32)
    # a padded tile leaves the tree unchanged bitwise
    x = np.array([-0.0, -0.0, 1.0], np.float32)
    t = tiles(x, 4, axis=0)
    assert t.shape == (1, 4) and np.signbit(t[0, 3])
    assert pairwise(t)[0] == 1.0
    y = np.array([-0.0, -0.0], np.float32)
    assert np.signbit(pairwise(tiles(y, 4, axis=0))[0])


def test_accumulate_one_rounding():
    out = np.array([1.0], np.float32)
    tot = np.array([2.0 ** -24 + 2.0 ** -25], np.float32)  # above half an ulp of 1
    assert accumulate(out, tot)[0] == np.float32(1.0 + 2.0 ** -23)
    # one add of the total is not the same as adding its pieces one by one
    pieces = np.array([2.0 ** -24, 2.0 ** -25], np.float32)
    stepwise = np.float32(np.float32(1.0 + pieces[0]) + pieces[1])
    assert stepwise == np.float32(1.0) != accumulate(out, pieces.sum(dtype=np.float32).reshape(1))[0]


def test_tiles_layout():
    x = np.arange(10, dtype=np.float32).reshape(5, 2)
    t = tiles(x, 4, axis=0)
    assert t.shape == (2, 2, 4)
    assert list(t[0, 1]) == [1, 3, 5, 7]
    assert t[1, 0, 0] == 8 and np.all(np.signbit(t[1, :, 1:]))


def test_widen_bf16_exact():
    bits = np.array([0x3F80, 0xBF80, 0x0001, 0x7F7F, 0x8000], np.uint16)
    v = widen_bf16(bits)
    assert v[0] == 1.0 and v[1] == -1.0 and v[2] == np.float32(2.0 ** -133)
    assert v[3] == np.float32(3.3895313892515355e38) and np.signbit(v[4]) and v[4] == 0
