"""ctypes loader of the oracle's C sources (test infrastructure only).

The shared objects are built by the build entry (gcc -O2 -ffp-contract=off
-fopenmp); if one is missing or older than its source, it is compiled here.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
GCC_FLAGS = ["-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared"]

_libs = {}


def build(name: str) -> str:
    src = os.path.join(HERE, name + ".c")
    out = os.path.join(HERE, name + ".so")
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", *GCC_FLAGS, src, "-o", tmp], check=True)
    os.replace(tmp, out)
    return out


def load(name: str) -> ctypes.CDLL:
    if name not in _libs:
        src = os.path.join(HERE, name + ".c")
        so = os.path.join(HERE, name + ".so")
        if not os.path.exists(so) or os.path.getmtime(so) < os.path.getmtime(src):
            build(name)
        _libs[name] = ctypes.CDLL(so)
    return _libs[name]


def threads() -> int:
    """Threads the OpenMP loops of the C oracle use (OMP_NUM_THREADS, else the CPUs this process may run on)."""
    v = os.environ.get("OMP_NUM_THREADS")
    if v and v.isdigit() and int(v) > 0:
        return int(v)
    return len(os.sched_getaffinity(0))
