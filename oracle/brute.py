"""Scalar, loop-by-loop restatements of the four cases for tiny inputs (pins only).

Written separately from the vectorised oracle modules: one Python loop per
index, ``np.float32`` scalars, the pairwise tree as recursive halving, the
stable sort as Python's ``sorted`` (which is stable). The vectorised oracle
must agree with these bit for bit. Test infrastructure only.
"""
from __future__ import annotations

import numpy as np

from . import detmath

F = np.float32
NZ = np.float32(-0.0)


def _w(bits) -> np.float32:
    return np.array([int(bits) << 16], np.uint32).view(np.float32)[0]


def _gate(v) -> np.float32:
    """An input element: a float32 value as is, else bf16 bits widened."""
    return v if isinstance(v, np.float32) else _w(v)


def tree(vals):
    """Recursive halving: tree(v) = tree(left half) + tree(right half)."""
    if len(vals) == 1:
        return F(vals[0])
    h = len(vals) // 2
    return F(tree(vals[:h]) + tree(vals[h:]))


def fold(vals):
    acc = NZ
    for v in vals:
        acc = F(acc + F(v))
    return acc


def padded_tiles(vals, block):
    out = []
    for s in range(0, len(vals), block):
        t = list(vals[s:s + block])
        t += [NZ] * (block - len(t))
        out.append(t)
    return out


def dprob(dprob0, dY, C, offs, tile_n=128):
    M = len(dprob0)
    out = [F(v) for v in dprob0]
    lo = min(max(int(offs[0]), 0), M)
    hi = min(max(int(offs[-1]), lo), M)
    for m in range(lo, hi):
        terms = []
        for n in range(len(dY[m])):
            c = _w(C[m][n])
            sq = F(c * c) if c > 0 else F(0.0)
            terms.append(F(_w(dY[m][n]) * sq))
        slots = [tree(t) for t in padded_tiles(terms, tile_n)]
        out[m] = F(out[m] + fold(slots))
    return np.array(out, np.float32)


def colsum(a, dg, A_log, dt_bias, dA0, ddt0, block_t):
    T, H = len(a), len(A_log)
    r1, r2 = [], []
    for h in range(H):
        nA = -detmath.exp32(np.float32(A_log[h]))[()]
        t1, t2 = [], []
        for t in range(T):
            x = F(_gate(a[t][h]) + F(dt_bias[h]))
            e = detmath.exp32(F(-abs(x)))[()]
            sp = detmath.softplus_from(np.float32(x), np.float32(e))[()]
            sg = detmath.sigmoid_from(np.float32(x), np.float32(e))[()]
            d = _gate(dg[t][h])
            t1.append(F(d * F(nA * sp)))
            t2.append(F(d * F(nA * sg)))
        r1.append(F(F(dA0[h]) + fold([tree(x) for x in padded_tiles(t1, block_t)])))
        r2.append(F(F(ddt0[h]) + fold([tree(x) for x in padded_tiles(t2, block_t)])))
    return np.array(r1, np.float32), np.array(r2, np.float32)


def index_add(out0, ids, src, chunk_rows):
    n_rows, D = len(out0), len(out0[0])
    out = [[F(v) for v in row] for row in out0]
    pairs = sorted([(int(i), p) for p, i in enumerate(ids) if 0 <= int(i) < n_rows], key=lambda t: t[0])
    runs = {}
    for i, p in pairs:
        runs.setdefault(i, []).append(p)
    for i, rows in runs.items():
        for d in range(D):
            parts = []
            for s in range(0, len(rows), chunk_rows):
                parts.append(fold([_gate(src[p][d]) for p in rows[s:s + chunk_rows]]))
            out[i][d] = F(out[i][d] + fold(parts))
    return np.array(out, np.float32)


def literal_sequential_index_add(out0, ids, src):
    """out[id] += src[p] one row at a time in stable id order (no chunks)."""
    n_rows = len(out0)
    out = np.array(out0, np.float32, copy=True)
    for i, p in sorted([(int(i), p) for p, i in enumerate(ids) if 0 <= int(i) < n_rows], key=lambda t: t[0]):
        for d in range(out.shape[1]):
            out[i, d] = F(out[i, d] + _gate(src[p][d]))
    return out


def indexer_dk(dk0, ids, predict, target, q, scale, chunk_rows):
    """Fused indexer dK, one slot at a time: kept targets clamped below at the float32 nearest e^-100 on
    valid slots, the row sum left to right, the slot coefficient, its source row c * q, then the chunked
    index_add above (ids, predict, target [Q][K]; q [Q][D] bf16 bits or float32 values)."""
    n_rows = len(dk0)
    e100 = np.array([27], np.uint32).view(np.float32)[0]
    Q, K = len(ids), len(ids[0])
    flat_ids, src = [], []
    for r in range(Q):
        valid = [0 <= int(ids[r][j]) < n_rows for j in range(K)]
        kept = [(F(target[r][j]) if F(target[r][j]) > e100 else e100) if valid[j] else F(0.0) for j in range(K)]
        S = fold(kept)
        for j in range(K):
            c = F(F(F(F(predict[r][j]) * S) - kept[j]) * F(scale)) if valid[j] else F(0.0)
            flat_ids.append(int(ids[r][j]))
            src.append([F(c * _gate(v)) for v in q[r]])
    return index_add(dk0, flat_ids, src, chunk_rows)


def wgrad_exact_integer(main_grad0, G, X, offs):
    """For small-integer inputs: main_grad0 + exact integer G_e^T X_e, per element."""
    E, M, N = np.shape(main_grad0)
    out = np.array(main_grad0, np.float32, copy=True)
    for e in range(E):
        for i in range(M):
            for j in range(N):
                s = 0
                for r in range(int(offs[e]), int(offs[e + 1])):
                    s += int(_w(G[r][i])) * int(_w(X[r][j]))
                out[e, i, j] = F(out[e, i, j] + F(s))
    return out


def dbias(dbias0, dA, offs, block_m):
    M = len(dA)
    N = len(dA[0]) if M else 0
    out = [[F(v) for v in row] for row in dbias0]
    b = []
    for e, o in enumerate(offs):
        lo = 0 if e == 0 else b[-1]
        b.append(min(max(int(o), lo), M))
    for e in range(len(b) - 1):
        if b[e + 1] <= b[e]:
            continue
        for n in range(N):
            col = [_w(dA[m][n]) for m in range(b[e], b[e + 1])]
            slots = [tree(t) for t in padded_tiles(col, block_m)]
            out[e][n] = F(out[e][n] + fold(slots))
    return np.array(out, np.float32).reshape(np.asarray(dbias0).shape)


def topk_canonical(ids, logits):
    """Per row: insertion sort of (id, slot) with padding last, then the softmax
    in that order, one scalar at a time."""
    Q, K = len(ids), len(ids[0])
    io = np.zeros((Q, K), np.int32); lo = np.zeros((Q, K), np.float32); po = np.zeros((Q, K), np.float32)
    for q in range(Q):
        order = []
        for j in range(K):
            key = (0 if int(ids[q][j]) >= 0 else 1, int(ids[q][j]) if int(ids[q][j]) >= 0 else 0, j)
            pos = len(order)
            while pos > 0 and order[pos - 1][0] > key:
                pos -= 1
            order.insert(pos, (key, j))
        for r, (_, j) in enumerate(order):
            io[q, r] = ids[q][j]; lo[q, r] = logits[q][j]
        nv = sum(1 for j in range(K) if int(ids[q][j]) >= 0)
        if nv == 0:
            continue
        m = lo[q, 0]
        for r in range(1, nv):
            m = lo[q, r] if lo[q, r] > m else m
        e = [detmath.exp32(np.float32(F(lo[q, r] - m)))[()] for r in range(nv)]
        S = fold(e)
        for r in range(nv):
            po[q, r] = F(F(e[r]) / S)
    return io, lo, po
