"""GPU parity of det_topk_canonicalize against the CPU oracle (bitwise): ids,
permuted logits and probabilities; slot-order invariance on the GPU."""
import numpy as np
import pytest

import deterministic_gradient_reductions_amd as dg
import workloads as W
from oracle import topk as ot
from tests.gpu_util import assert_bitwise, dev_f32, dev_i32, host, note

pytestmark = pytest.mark.gpu


def run(ids, logits, out_pad=0):
    import torch
    Q, K = ids.shape
    i, l = dev_i32(ids), dev_f32(logits)
    io = torch.full((Q, K + out_pad), 7, dtype=torch.int32, device="cuda")[:, :K]
    lo = torch.full((Q, K + out_pad), 7.0, dtype=torch.float32, device="cuda")[:, :K]
    po = torch.full((Q, K + out_pad), 7.0, dtype=torch.float32, device="cuda")[:, :K]
    torch.cuda.synchronize()
    dg.det_topk_canonicalize(i, l, io, lo, po)
    return host(io), host(lo), host(po)


def check(ids, logits, what, out_pad=0):
    got = run(ids, logits, out_pad)
    want = ot.canonicalize(ids, logits)
    assert np.array_equal(got[0], want[0]), what + " ids"
    assert_bitwise(got[1], want[1], what + " logits")
    assert_bitwise(got[2], want[2], what + " probs")


@pytest.mark.parametrize("Q,K,n_keys,distinct,pad", [(64, 512, 8192, True, 0.05), (33, 1000, 4096, True, 0.1),
                                                     (50, 64, 100, False, 0.3), (7, 1, 5, False, 0.5),
                                                     (20, 129, 300, False, 0.0), (9, 1024, 2000, True, 0.02),
                                                     (12, 37, 20, False, 0.2), (16, 37, 5000, True, 0.2),
                                                     (16, 100, 300, True, 0.1)])
def test_parity(Q, K, n_keys, distinct, pad):
    note("topk parity Q=%d K=%d distinct=%s pad=%.2f" % (Q, K, distinct, pad))
    inp = W.topk_inputs(Q=Q, K=K, n_keys=n_keys, seed=K, distinct=distinct, pad_frac=pad)
    ids = inp.ids.copy()
    ids[0, :] = -1  # a row that is all padding
    check(ids, inp.logits, "topk", out_pad=3 if K % 2 else 0)


@pytest.mark.parametrize("top", [(1 << 21) - 2, (1 << 21) - 1, 2**31 - 1])
def test_id_range(top):
    """Ids up to the largest one the 32-bit sort key holds, and past it (the
    64-bit key); rows of both kinds share workgroups."""
    note("topk id range top=%d" % top)
    inp = W.topk_inputs(Q=41, K=300, n_keys=64, seed=3, distinct=False, pad_frac=0.1)
    ids = inp.ids.copy()
    ids[ids >= 0] += top - 63
    ids[1::3] = np.where(ids[1::3] >= 0, ids[1::3] - (top - 63), -1)  # small ids on every third row
    ids[2, :] = -1
    check(ids, inp.logits, "topk ids to %d" % top)


def test_padding_keeps_its_own_negative_id():
    """Every negative id is padding and comes out unchanged, in slot order after the valid ids:
    -1, -2, -1000 and INT32_MIN mixed in one row, rows of 32- and 64-bit keys."""
    inp = W.topk_inputs(Q=24, K=200, n_keys=3000, seed=11, distinct=True, pad_frac=0.0)
    ids = inp.ids.copy()
    rng = np.random.default_rng(5)
    neg = np.array([-1, -2, -1000, np.iinfo(np.int32).min], np.int32)
    mask = rng.random(ids.shape) < 0.15
    ids[mask] = neg[rng.integers(0, 4, size=int(mask.sum()))]
    ids[3, ::2] = np.where(ids[3, ::2] >= 0, ids[3, ::2] + (1 << 22), ids[3, ::2])  # a row with 64-bit keys
    ids[4, :] = neg[rng.integers(0, 4, size=200)]                                 # a row of padding only
    note("topk negative padding ids")
    check(ids, inp.logits, "topk negative padding")


def test_counting_window_edges():
    """Rows whose distinct valid ids span exactly 16384 values (the widest span
    counted from the id bitmap) and 16385 (sorted), at base 0 and at 2^24; a
    narrow row with one repeated id (sorted); all of them sharing workgroups
    with ordinary rows."""
    inp = W.topk_inputs(Q=16, K=512, n_keys=8192, seed=13, distinct=True, pad_frac=0.05)
    ids = inp.ids.copy()
    rng = np.random.default_rng(17)
    for q, base, top in [(0, 0, 16383), (1, 0, 16384), (2, 1 << 24, 16383), (3, 1 << 24, 16384), (4, 5, 300000),
                         (9, (1 << 31) - 16384, 16383)]:
        valid = ids[q] >= 0
        n = int(valid.sum())
        vals = np.concatenate([[0, top], rng.choice(np.arange(1, top), n - 2, replace=False)])
        ids[q, valid] = (base + rng.permutation(vals)).astype(np.int32)
    v = np.flatnonzero(ids[5] >= 0)
    ids[5, v[-1]] = ids[5, v[0]]  # a repeated id
    note("topk counting window edges")
    check(ids, inp.logits, "topk window edges")


def test_full_size_and_slot_order_invariance():
    inp = W.topk_inputs(seed=7)  # 4096 x 512
    note("topk full size")
    ref = run(inp.ids, inp.logits)
    want = ot.canonicalize(inp.ids, inp.logits)
    assert np.array_equal(ref[0], want[0])
    assert_bitwise(ref[1], want[1], "topk full logits"); assert_bitwise(ref[2], want[2], "topk full probs")
    perm = np.argsort(np.random.default_rng(1).random(inp.ids.shape), axis=1)
    got = run(np.take_along_axis(inp.ids, perm, 1), np.take_along_axis(inp.logits, perm, 1))
    valid = ref[0] >= 0
    assert np.array_equal(got[0], ref[0])
    assert_bitwise(got[2], ref[2], "probs after reshuffle")
    assert np.array_equal(got[1].view(np.uint32)[valid], ref[1].view(np.uint32)[valid])


def test_replay_under_load():
    """20 calls at 4096 x 512 while a side stream streams HBM: identical bits every time."""
    import torch
    from tests.gpu_util import SideLoad
    inp = W.topk_inputs(seed=7)
    i, l = dev_i32(inp.ids), dev_f32(inp.logits)
    io, lo, po = torch.empty_like(i), torch.empty_like(l), torch.empty_like(l)
    load = SideLoad()
    pats = set()
    for r in range(20):
        load.kick()
        dg.det_topk_canonicalize(i, l, io, lo, po)
        pats.add(host(io).tobytes() + host(lo).tobytes() + host(po).tobytes())
    load.wait()
    assert len(pats) == 1
