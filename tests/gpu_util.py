"""Helpers for the GPU parity tests: upload seeded host arrays, compare bits,
and keep a second stream busy while a deterministic call runs."""
from __future__ import annotations

import sys

import numpy as np


def torch():
    import torch as _t
    return _t


def dev_bf16(bits: np.ndarray):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(t.bfloat16)


def dev_f32(x: np.ndarray):
    return torch().from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def dev_i32(x: np.ndarray):
    return torch().from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()


def host(t) -> np.ndarray:
    torch().cuda.synchronize()
    return t.detach().cpu().numpy()


def bits(x) -> np.ndarray:
    return np.asarray(x, np.float32).view(np.uint32)


def assert_bitwise(got, want, what=""):
    g, w = bits(got), bits(want)
    if not np.array_equal(g, w):
        bad = np.nonzero(g.ravel() != w.ravel())[0]
        i = bad[0]
        raise AssertionError("%s: %d of %d elements differ; first at flat %d: got %r want %r" % (
            what, len(bad), g.size, i, np.asarray(got).ravel()[i], np.asarray(want).ravel()[i]))


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64); b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def note(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


class SideLoad:
    """Streams HBM traffic on a separate stream (default priority) while active."""

    def __init__(self, mib: int = 256, iters: int = 8):
        t = torch()
        self.stream = t.cuda.Stream()
        self.a = t.empty(mib * 1024 * 1024 // 4, dtype=t.float32, device="cuda").uniform_()
        self.b = t.empty_like(self.a)
        self.iters = iters

    def kick(self) -> None:
        t = torch()
        with t.cuda.stream(self.stream):
            for _ in range(self.iters):
                self.b.copy_(self.a)
                self.a.mul_(1.0000001)

    def wait(self) -> None:
        self.stream.synchronize()
