"""The determinism manifest (tests/manifest.py) covers every accumulating entry
point declared in include/detgrad.h, and every test it names exists."""
import ast
import os
import re

from tests.manifest import MANIFEST, NOT_ENTRY_POINTS

HERE = os.path.dirname(os.path.abspath(__file__))
HEADER = os.path.join(os.path.dirname(HERE), "include", "detgrad.h")


def declared():
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    return set(re.findall(r"\b(det_[a-z0-9_]+)\s*\(", src))


def test_every_entry_point_is_listed():
    entries = {n for n in declared() if not n.endswith("_workspace_size")} - NOT_ENTRY_POINTS
    assert entries == set(MANIFEST), (entries ^ set(MANIFEST))


def test_every_listed_test_exists():
    defs = {}
    for f in os.listdir(HERE):
        if f.endswith(".py"):
            tree = ast.parse(open(os.path.join(HERE, f)).read())
            defs[f] = {n.name for n in tree.body if isinstance(n, ast.FunctionDef)}
    for name, e in MANIFEST.items():
        assert e["cite"] and e["graph"]
        for kind in ("replay", "parity", "atomic", "graph"):
            for t in e[kind] or []:
                f, fn = t.split("::")
                assert fn in defs.get(f, set()), "%s: %s missing" % (name, t)
