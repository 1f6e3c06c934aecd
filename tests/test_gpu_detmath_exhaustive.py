"""Every float32 input of the gate's exp, softplus and sigmoid sequences: the
device's bits against the CPU oracle's (oracle/detmath.py), NaN payloads
aside. The 2^32 inputs go in 64 chunks of 2^26; by default every 8th chunk
runs (a spread of 2^29 inputs over every exponent), and DETGRAD_EXHAUSTIVE=1
runs all 64."""
import concurrent.futures as cf
import os
import time

import numpy as np
import pytest

import deterministic_gradient_reductions_amd as dg
from oracle import _cmodel, detmath as dm
from tests.gpu_util import note

pytestmark = pytest.mark.gpu

CHUNK = 1 << 26
ALL = os.environ.get("DETGRAD_EXHAUSTIVE", "") == "1"
CHUNKS = list(range(64)) if ALL else list(range(0, 64, 8))


def oracle_bits(fn, x, pool, n):
    parts = np.array_split(np.arange(x.size), n)

    def one(idx):
        with np.errstate(all="ignore"):
            return getattr(dm, fn)(x[idx[0]:idx[-1] + 1])
    return np.concatenate(list(pool.map(one, parts))).view(np.uint32)


@pytest.mark.parametrize("fn", ["exp32", "softplus32", "sigmoid32"])
def test_every_float32_input(fn):
    import torch
    n = _cmodel.threads()
    xd = torch.empty(CHUNK, dtype=torch.float32, device="cuda")
    yd = torch.empty_like(xd)
    base = torch.arange(CHUNK, dtype=torch.int64, device="cuda")
    t0 = time.time()
    bad = 0
    first = None
    with cf.ThreadPoolExecutor(n) as pool:
        for c in CHUNKS:
            # bit patterns c * 2^26 .. (c + 1) * 2^26 - 1, made on the device
            xd.view(torch.int32).copy_((base + c * CHUNK).to(torch.int32) if c < 32 else
                                       (base + c * CHUNK - (1 << 32)).to(torch.int32))
            dg.det_detmath_eval(xd, yd, fn)
            torch.cuda.synchronize()
            x = xd.cpu().numpy()
            g = yd.cpu().numpy().view(np.uint32)
            w = oracle_bits(fn, x, pool, n)
            nan = ((g & 0x7F800000) == 0x7F800000) & ((g & 0x7FFFFF) != 0) & \
                  ((w & 0x7F800000) == 0x7F800000) & ((w & 0x7FFFFF) != 0)
            diff = np.nonzero((g != w) & ~nan)[0]
            bad += len(diff)
            if len(diff) and first is None:
                first = (x[diff[0]], g[diff[0]], w[diff[0]])
    note("detmath %s: %d of %d float32 inputs checked (%d chunks), %d differ, %.0f s, %d threads" % (
        fn, len(CHUNKS) * CHUNK, 1 << 32, len(CHUNKS), bad, time.time() - t0, n))
    assert bad == 0, "first mismatch x=%r gpu=%#x cpu=%#x" % first
