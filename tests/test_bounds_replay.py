"""CPU replay of the kernels' global-memory index arithmetic at full size.

Each replay restates, in numpy, the index expressions and guards of one
kernel (the same names as in its source: workgroup, wave, lane, tile, piece)
and evaluates them for every workgroup and lane of the launch that the host
code makes for the full-size workloads (and for ragged variants of them).
Every element index a kernel can form behind its guards must lie inside the
buffer it addresses; accesses through a buffer resource are range-checked by
the hardware, so for those the replay checks that the resource's byte range
lies inside its tensor. No GPU is involved: a failing case here names an
out-of-range access before a kernel is ever launched with it.
"""
import numpy as np
import pytest

import workloads as W
from oracle import index_add as oi

WG = 256


def inside(name, idx, size):
    idx = np.asarray(idx)
    if idx.size == 0:
        return
    lo, hi = int(idx.min()), int(idx.max())
    assert 0 <= lo and hi < size, "%s: indices [%d, %d] outside [0, %d)" % (name, lo, hi, size)


def cdiv(a, b):
    return -(-a // b)


# ------------------------------------------------------------------ colsum
def colsum_order(T, H, BT, BH):
    """colsum_kernel's workgroup order: a 1-D grid of groups of 8 tiles times the head
    groups; workgroup u = 8 * HG * c + 8 * j + x takes tile 8c + x and head group j and
    exits when that tile is past the end. Returns (tile, head group) per workgroup, -1
    for the exiting ones."""
    S, HG = cdiv(T, BT), cdiv(H, BH)
    u = np.arange(cdiv(S, 8) * 8 * HG, dtype=np.int64)
    per = 8 * HG
    r = u % per
    tile = (u // per) * 8 + (r & 7)
    hg = r >> 3
    live = tile < S
    return np.where(live, tile, -1), np.where(live, hg, -1)


def test_colsum_order_covers_every_tile_once():
    for T, H, BT, BH in [(16384, 32, 64, 8), (16323, 32, 256, 32), (4133, 17, 128, 16), (100, 5, 64, 8),
                         (4194304, 32, 256, 8), (64 * 9, 40, 64, 8)]:
        tile, hg = colsum_order(T, H, BT, BH)
        S, HG = cdiv(T, BT), cdiv(H, BH)
        live = tile >= 0
        pairs = tile[live] * HG + hg[live]
        assert np.array_equal(np.sort(pairs), np.arange(S * HG)), (T, H, BT, BH)
        # the head groups of one tile sit on one XCD (u % 8) and run back to back
        u = np.nonzero(live)[0]
        assert np.all((u % 8) == (tile[live] % 8))


def replay_colsum(T, H, BT, BH, tiles=None, dg_view=True):
    """colsum_kernel<R, BH> and colsum_fold_kernel; a is [T, H] contiguous, dg the
    [T, 2H] base tensor viewed from column H (the gate backward's layout). The
    workgroup order is colsum_order's (checked to cover every (tile, head group)
    once), so the replay walks tiles and head groups directly."""
    R = BT * BH // WG
    kBT, S = R * WG // BH, cdiv(T, BT)
    assert kBT == BT
    tiles = np.arange(S) if tiles is None else np.asarray(tiles)
    tid = np.arange(WG)
    hl, rb = tid % BH, tid // BH
    for by in range(cdiv(H, BH)):
        h = by * BH + hl                                                    # [WG]
        r0 = tiles[:, None] * kBT + rb[None, :] * R                         # [tiles, WG]
        t = r0[:, :, None] + np.arange(R)[None, None, :]                    # [tiles, WG, R]
        ok = (h[None, :, None] < H) & (t < T)
        hh = np.broadcast_to(h[None, :, None], t.shape)
        inside("colsum a", (t * H + hh)[ok], T * H)
        dgo = H if dg_view else 0
        dgs = 2 * H if dg_view else H
        inside("colsum dg", (dgo + t * dgs + hh)[ok], T * dgs)
        inside("colsum A_log/dt_bias", h[h < H], H)
        # slot writes by the first BH threads
        lead = (tid < BH) & (h < H)
        inside("colsum slot", (tiles[:, None] * H + h[None, :])[:, lead], S * H)
    # fold: wave per (head, gradient); lane j reads tiles i0 + j + 64 q < S
    i0 = np.arange(0, S, 256)
    i = (i0[:, None, None] + np.arange(64)[None, :, None] + 64 * np.arange(4)[None, None, :]).ravel()
    i = i[i < S]
    for hv in (0, H - 1):
        inside("colsum fold", i * H + hv, S * H)


@pytest.mark.parametrize("T,H", [(16384, 32), (16323, 32), (4096, 16), (4133, 17)])
@pytest.mark.parametrize("BT,BH", [(bt, bh) for bt in (64, 128, 256) for bh in (8, 16, 32)])
def test_colsum(T, H, BT, BH):
    replay_colsum(T, H, BT, BH)


def test_colsum_bandwidth_companion():
    """T = 4,194,304 x H = 32 at its tile 256 x 8: the first and last tiles and every 97th in between."""
    T, H, BT, BH = 4194304, 32, 256, 8
    S = cdiv(T, BT)
    tiles = np.unique(np.concatenate([np.arange(4), np.arange(S - 4, S), np.arange(0, S, 97)]))
    replay_colsum(T, H, BT, BH, tiles)


# ------------------------------------------------------------------ dprob
def valid_rows(offs, M):
    a, b = int(offs[0]), int(offs[-1])
    lo = min(max(a, 0), M)
    return lo, min(max(b, lo), M)


def replay_dprob(M, N, offs, rows_per_wg=4, ld=None):
    ld = N if ld is None else ld
    lo, hi = valid_rows(offs, M)
    n_chunks = cdiv(N, 512)
    lane = np.arange(64)
    # deterministic arm: grid ceil(M / rows_per_wg); wave w takes rows first + w, first + w + 4, ...
    b = np.arange(cdiv(M, rows_per_wg))
    first = lo + b * rows_per_wg
    end = np.minimum(first + rows_per_wg, hi)
    m = (first[:, None] + np.arange(rows_per_wg)[None, :])
    m = m[m < end[:, None]]
    ch = np.arange(n_chunks)
    col = ch[:, None] * 512 + 8 * lane[None, :]
    col = col[col < N]
    inside("dprob rows", m, M)
    if m.size:
        inside("dprob dY/C", np.array([m.min() * ld + col.min(), m.max() * ld + col.max() + 7]), M * ld)
    # atomic arm: wave w of rows * n_chunks, row-major
    rows = hi - lo
    waves = np.arange(cdiv(M * n_chunks, 4) * 4)
    waves = waves[waves < rows * n_chunks]
    ma, cha = lo + waves // n_chunks, waves % n_chunks
    inside("dprob atomic rows", ma, M)
    ca = cha * 512
    assert (ca < N).all()


@pytest.mark.parametrize("rpw", [1, 4, 7, 64])
def test_dprob(rpw):
    counts = W.expert_counts(16384, 8, 256, 4, 0)
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    replay_dprob(16384, 2048, offs, rpw)
    # offsets past M and a shorter last expert: rows clamp to [0, M)
    replay_dprob(16000, 2048, offs, rpw)
    replay_dprob(5000, 1000, np.array([-3, 700, 2900, 5100]), rpw, ld=1008)


# ------------------------------------------------------------------ dbias
def expert_table(offs, M, bm):
    """b_e clamped monotone; tiles per expert and their first global tile."""
    b = np.minimum(np.maximum.accumulate(np.maximum(np.asarray(offs, np.int64), 0)), M)
    nt = np.where(b[1:] > b[:-1], cdiv(b[1:] - b[:-1], bm), 0)
    first = np.concatenate([[0], np.cumsum(nt)])
    return b, nt, first


def replay_dbias(M, N, offs, bm, lda=None, past_end_row="quarter", bn=512):
    """past_end_row: the row a load takes once it lies past the tile end; "quarter" is the
    kernel's rule (the quarter's first row), "piece" the piece's own first row. bn: columns
    per workgroup, bn / 64 per lane."""
    lda = N if lda is None else lda
    E = len(offs) - 1
    Q, P = bm // 4, 16
    NP = Q // P
    cpl = bn // 64
    ncb = cdiv(N, bn)
    max_tiles = cdiv(M, bm) + E
    b, nt, first = expert_table(offs, M, bm)
    lane, wave = np.arange(64), np.arange(4)
    for t in range(int(first[-1])):
        e = int(np.searchsorted(first, t, side="right") - 1)
        r0 = int(b[e] + (t - first[e]) * bm)
        r1 = min(r0 + bm, int(b[e + 1]))
        assert 0 <= r0 < r1 <= M
        a0 = r0 + wave * Q                                                  # [4]
        for w in range(4):
            if a0[w] >= r1:
                continue
            # load_piece: row a + i, or the quarter's first row once past r1
            a = a0[w] + np.arange(NP)[:, None] * P + np.arange(P)[None, :]
            safe = a0[w] if past_end_row == "quarter" else (a0[w] + np.arange(NP)[:, None] * P)
            r = np.where(a < r1, a, safe)
            inside("dbias dA rows (tile %d)" % t, r, M)
        for cb in range(ncb):
            col = cb * bn + cpl * lane
            col = col[col < N]
            assert (col + cpl - 1 < N).all()
            inside("dbias slot", t * N + col, max_tiles * N)
    # fold: slots of an expert's tiles, tstart has E + 1 entries
    inside("dbias fold tiles", np.arange(int(first[-1])), max_tiles)
    if first[-1]:
        inside("dbias dA extent", np.array([(M - 1) * lda + N - 1]), M * lda)


@pytest.mark.parametrize("bn", [512, 256, 128])
@pytest.mark.parametrize("bm", [64, 128, 256])
def test_dbias(bm, bn):
    counts = W.expert_counts(16384, 8, 256, 6, 0)
    offs = np.concatenate([[0], np.cumsum(counts)])
    replay_dbias(16384, 2048, offs, bm, bn=bn)
    # ragged: tiles that end inside a quarter, an empty expert, offsets past M
    replay_dbias(3001, 520, np.array([0, 10, 10, 1000, 2999, 3500]), bm, lda=528, bn=bn)


def test_dbias_replay_catches_a_piece_row_past_m():
    """A load that takes its piece's own first row once the piece lies past the tile end reads
    past M in the last tile of a short last expert (the replay must reject that rule)."""
    with pytest.raises(AssertionError, match="dbias dA rows"):
        replay_dbias(3001, 520, np.array([0, 10, 10, 1000, 2999, 3500]), 256, lda=528, past_end_row="piece")


# ------------------------------------------------------------------ wgrad
XCDS = 8


def plan_xcds(tiles_m, tiles_n, block_m, block_n):
    best, xm, xn = -1, 0, 0
    pm = 1
    while pm <= XCDS:
        pn = XCDS // pm
        if pm <= tiles_m and pn <= tiles_n:
            by = cdiv(tiles_m, pm) * block_m * 2 + cdiv(tiles_n, pn) * block_n * 2
            if best < 0 or by < best:
                best, xm, xn = by, pm, pn
        pm *= 2
    return xm, xn


def unit_of(u, tiles_m, tiles_n, xm, xn, max_splits):
    if xm > 0:
        x, slot = u % XCDS, u // XCDS
        am, an = x // xn, x % xn
        mlo, mhi = am * tiles_m // xm, (am + 1) * tiles_m // xm
        nlo, nhi = an * tiles_n // xn, (an + 1) * tiles_n // xn
        per = (mhi - mlo) * (nhi - nlo)
        if per == 0:
            return None
        q = slot // per
        if q >= max_splits:
            return None
        t = slot % per
        return q, mlo + t // (nhi - nlo), nlo + t % (nhi - nlo)
    tiles = tiles_m * tiles_n
    q = u // tiles
    if q >= max_splits:
        return None
    t = u % tiles
    return q, t // tiles_n, t % tiles_n


def splits_by_size(offs, T_total, split_rows):
    """Split list in the kernel's size order: experts by decreasing rows (ties by index), each
    expert's splits ascending; with the natural index g (expert order, then split order)."""
    E = len(offs) - 1
    b = np.minimum(np.maximum.accumulate(np.maximum(np.asarray(offs, np.int64), 0)), T_total)
    te = b[1:] - b[:-1]
    se = np.where(te <= 0, 0, 1 if split_rows == 0 else cdiv(te, max(split_rows, 1)))
    gs = np.concatenate([[0], np.cumsum(se)])
    order = sorted(range(E), key=lambda e: (-te[e], e))
    out = []
    for e in order:
        for s in range(int(se[e])):
            r0 = int(b[e]) if split_rows == 0 else int(b[e]) + s * split_rows
            r1 = int(b[e + 1]) if split_rows == 0 else min(r0 + split_rows, int(b[e + 1]))
            out.append((e, int(gs[e]) + s, int(se[e]), r0, r1))
    return out


def replay_wgrad(offs, M, N, ktiles_per_split, ldg=None, ldx=None, ld_m=None):
    ldg, ldx = ldg or M, ldx or N
    ld_m = ld_m or N
    E, T = len(offs) - 1, int(offs[-1])
    split_rows = 0 if ktiles_per_split == 0 else 512 * ktiles_per_split
    max_splits = E if ktiles_per_split == 0 else cdiv(T, split_rows) + E
    tiles_m, tiles_n = cdiv(M, 256), N // 256
    xm, xn = plan_xcds(tiles_m, tiles_n, 256, 256)
    if xm > 0:
        per_max = max(((x // xn + 1) * tiles_m // xm - (x // xn) * tiles_m // xm) *
                      ((x % xn + 1) * tiles_n // xn - (x % xn) * tiles_n // xn) for x in range(XCDS))
        n_units = XCDS * per_max * max_splits
    else:
        n_units = tiles_m * tiles_n * max_splits
    sp = splits_by_size(offs, T, split_rows)
    lane = np.arange(64)
    r, kg = lane & 31, lane >> 5
    c = np.arange(16)
    i, j = np.arange(4), np.arange(4)
    seen = set()
    for u in range(n_units):
        un = unit_of(u, tiles_m, tiles_n, xm, xn, max_splits)
        if un is None:
            continue
        q, mt, nt = un
        if q >= len(sp):
            continue
        e, g, n_split, r0, r1 = sp[q]
        seen.add((q, mt, nt))
        rows = r1 - r0
        assert 0 <= r0 < r1 <= T and e < E and g < max_splits
        # buffer resources: [r0 * ld * 2, (r0 + rows) * ld * 2) inside G [T, ldg] and X [T, ldx]
        assert (r0 + rows) * ldg * 2 <= T * ldg * 2 and (r0 + rows) * ldx * 2 <= T * ldx * 2
        assert (T + 512) * max(ldg, ldx) * 2 < 2 ** 31
        m0, n0 = mt * 256, nt * 256
        for wm in range(2):
            if m0 + 128 * wm >= M:
                continue                                                    # a wave past M stores nothing
            for wn in range(2):
                mw, nw = m0 + 128 * wm, n0 + 128 * wn
                row = (mw + 32 * i[:, None, None] + 8 * (c[None, :, None] // 4) + 4 * kg[None, None, :]
                       + c[None, :, None] % 4)
                col = nw + 32 * j[:, None] + r[None, :]
                inside("wgrad epilogue rows", row, M)
                inside("wgrad epilogue cols", col, N)
                if n_split == 1:
                    inside("wgrad main_grad", np.array([e * M * ld_m + row.max() * ld_m + col.max()]), E * M * ld_m)
                else:
                    inside("wgrad scratch", np.array([g * M * N + row.max() * N + col.max()]), max_splits * M * N)
    # every (split, tile) pair is computed exactly once
    assert len(seen) == len(sp) * tiles_m * tiles_n


@pytest.mark.parametrize("kps", [0, 2, 4])
def test_wgrad_headline(kps):
    wg = W.wgrad_tokens(8, seed=5)
    offs = np.concatenate([[0], np.cumsum(wg)])
    replay_wgrad(offs, 1408, 2048, kps)


def test_wgrad_ragged():
    replay_wgrad(np.array([0, 0, 37, 2049, 2049, 3100]), 384, 1024, 0, ldg=392, ldx=1032, ld_m=1040)
    replay_wgrad(np.array([0, 0, 37, 2049, 2049, 3100]), 384, 1024, 2, ldg=392, ldx=1032)


# ------------------------------------------------------------------ top-k
def test_topk():
    tk = W.topk_inputs(seed=7)
    Q, K = tk.ids.shape
    ids = tk.ids
    # sort keys (id or 2^31 for padding, slot): the first K sorted keys are the row's own slots
    hi = np.where(ids >= 0, ids.astype(np.int64), 2 ** 31)
    key = (hi << 32) | np.arange(K)[None, :]
    slot = (np.sort(key, axis=1) & 0xFFFFFFFF)
    inside("topk slot gather", slot, K)
    # narrow keys (id << 10 | slot) need ids below 2^21 - 1 and K <= 1024
    assert K <= 1024
    # wave w of workgroup b takes row 4 b + w; rows past Q load row 0 and store nothing
    for QQ in (Q, 1, 7, 8, 9, 4097):
        b, w = np.meshgrid(np.arange(cdiv(QQ, 4)), np.arange(4), indexing="ij")
        rows = (4 * b + w).ravel()
        assert np.array_equal(np.sort(rows[rows < QQ]), np.arange(QQ))  # every row exactly once
        inside("topk rows", np.where(rows < QQ, rows, 0), QQ)


def topk_count_positions(row, K, window=16384):
    """The counting path of the top-k kernel restated: None when the row is sorted instead
    (a repeated valid id, or valid ids spanning more than `window` values), else every
    slot's position, with the bitmap word indices checked against the bitmap."""
    v = row >= 0
    nv = int(v.sum())
    pos = np.empty(K, np.int64)
    if nv:
        ids = row[v].astype(np.int64)
        lo, hi = ids.min(), ids.max()
        if hi - lo >= window:
            return None
        b = ids - lo
        if np.unique(b).size != nv:
            return None
        w = b >> 5
        inside("topk bitmap words", w, window // 32)
        bm = np.zeros(window // 32, np.uint32)
        np.bitwise_or.at(bm, w, (np.uint32(1) << (b & 31).astype(np.uint32)))
        cnt = np.bitwise_count(bm).astype(np.int64)
        # lane l owns words 8 l .. 8 l + 7: the lane totals' exclusive wave scan, then a running sum
        lane_tot = cnt.reshape(64, 8).sum(1)
        lane_pre = np.cumsum(lane_tot) - lane_tot
        pre = (lane_pre[:, None] + np.cumsum(cnt.reshape(64, 8), 1) - cnt.reshape(64, 8)).ravel()
        below = np.bitwise_count(bm[w] & ((np.uint32(1) << (b & 31).astype(np.uint32)) - np.uint32(1)))
        pos[v] = pre[w] + below
    pos[~v] = nv + np.cumsum(~v)[~v] - 1
    inside("topk positions", pos, K)
    return pos


def test_topk_counting_positions():
    """The counting placement gives every slot of the workload's rows (and of edge rows) a
    distinct position inside the row, and the ids land in the canonical order."""
    tk = W.topk_inputs(seed=7)
    Q, K = tk.ids.shape
    rng = np.random.default_rng(3)
    edge = []
    for lo, span in [(0, 16383), (0, 16384), (1 << 24, 16383), ((1 << 31) - 16384, 16383)]:
        r = tk.ids[0].copy()
        vals = np.concatenate([[0, span], rng.choice(np.arange(1, span), int((r >= 0).sum()) - 2, replace=False)])
        r[r >= 0] = lo + rng.permutation(vals)
        edge.append(r)
    dup = tk.ids[1].copy()
    vi = np.flatnonzero(dup >= 0)
    dup[vi[-1]] = dup[vi[0]]
    edge += [dup, np.full(K, -1, np.int32)]
    counted = 0
    for row in list(tk.ids) + edge:
        pos = topk_count_positions(row, K)
        hi = np.where(row >= 0, row.astype(np.int64), 2 ** 31).astype(np.uint64)
        canon = row[np.argsort((hi << np.uint64(32)) | np.arange(K, dtype=np.uint64))]
        if pos is None:
            continue
        counted += 1
        assert np.array_equal(np.sort(pos), np.arange(K))
        placed = np.empty(K, row.dtype)
        placed[pos] = row
        assert np.array_equal(placed, canon)
    assert counted == Q + 4  # every workload row, the two in-window edge rows per base and the all-padding row
    assert topk_count_positions(edge[1], K) is None and topk_count_positions(dup, K) is None


# ------------------------------------------------------------------ index_add / indexer dK
def replay_index_add(ids, n_rows, dim, L, Q=None, K=None):
    """Descriptors, gather reads, scratch slots and fold reads of det_index_add (and the
    fused indexer dK, whose source rows are the query rows pos // K)."""
    ids = np.asarray(ids, np.int64).ravel()
    n_src = ids.size
    valid = (ids >= 0) & (ids < n_rows)
    cnt = np.bincount(ids[valid], minlength=n_rows).astype(np.int64)
    seg = np.concatenate([[0], np.cumsum(cnt)])
    n_valid = int(seg[-1])
    nc, fc = cdiv(cnt, L), cnt // L
    chk = np.concatenate([[0], np.cumsum(nc)])
    ful = np.concatenate([[0], np.cumsum(fc)])
    n_full = int(ful[-1])
    max_chunks = n_src // L + min(n_rows, n_src) + 1
    assert int(chk[-1]) <= max_chunks
    # the stable scatter: destination of position p = seg[id] + earlier positions with the same id
    perm, counts = oi.stable_order(ids, n_rows)
    assert (counts == cnt).all() and perm.size == n_valid
    inside("index_add perm", np.arange(n_valid), n_src)
    assert (ids[perm] == np.repeat(np.arange(n_rows), cnt)).all()
    # descriptors: chunk i of id k
    k = np.repeat(np.arange(n_rows), nc)
    i = np.arange(int(chk[-1])) - np.repeat(chk[:-1], nc)
    r0 = seg[k] + i * L
    s1 = np.minimum(seg[k] + cnt[k], n_src)
    ln = np.where(r0 + L < s1, L, np.maximum(s1 - r0, 0))
    at = np.where(ln == L, ful[k] + i, n_full + (chk[k] - ful[k]))
    slot = np.where(nc[k] == 1, -1, chk[k] + i)
    inside("index_add descriptor slot", at, max_chunks)
    assert np.unique(at).size == at.size
    assert (ln >= 1).all() and (r0 + ln <= n_valid).all()
    inside("index_add scratch slot", slot[slot >= 0], max_chunks)
    # gather: perm entry r0 + 64 w + lane inside the chunk, else r0 (a valid entry)
    inside("index_add gather perm", r0, n_src)
    inside("index_add gather perm end", r0 + ln - 1, n_src)
    pos = perm
    if K is None:
        inside("index_add src rows", pos, n_src)
    else:
        inside("indexer_dk query rows", pos // K, Q)
        inside("indexer_dk coef slots (scatter, by slot)", pos, n_src)
        # the gather reads (slot, coefficient) pairs in the sorted order: entries r0 .. r0 + len - 1
        inside("indexer_dk sorted pairs", np.concatenate([r0, r0 + ln - 1]), n_src)
    inside("index_add out rows", k[slot < 0], n_rows)
    # fold: the chunk partials of every id with more than one chunk
    multi = nc > 1
    inside("index_add fold", np.concatenate([np.arange(chk[kk], chk[kk + 1]) for kk in np.nonzero(multi)[0]] or
                                            [np.zeros(0, np.int64)]), max_chunks)


def replay_sort(ids, n_rows):
    """LDS and global indices of the count and scatter kernels (blocks of 4096 positions, 1024 threads,
    NW walking sub-blocks), and the destination each position gets from the kernel's decomposition
    (segment offset + earlier segments + earlier blocks + earlier sub-blocks + running count + rank),
    which must be the position's place in the stable order."""
    ids = np.asarray(ids, np.int64).ravel()
    n_src = ids.size
    B, T, SEG = 4096, 1024, 16
    nblk = cdiv(n_src, B)
    nseg = cdiv(nblk, SEG)
    hist_ld = cdiv(n_rows, 8) * 8
    pad = cdiv(n_rows, 4) * 4
    nw = next((w for w in (4, 2) if w * pad * 4 + B * 4 <= 80 * 1024), 1)
    bps = (B // 64) // nw
    assert nw * pad * 4 + B * 4 <= 160 * 1024
    # count: positions p0 + tid + 1024 u, u < 4; LDS histogram entries [0, hist_ld); row stores hist_ld / 8 vectors
    p = np.arange(n_src)
    valid = (ids >= 0) & (ids < n_rows)
    inside("count lds", ids[valid], hist_ld)
    inside("count hist row", np.array([0, nblk * hist_ld - 1]), nblk * hist_ld)
    # scatter: wave w takes batches w + 16 q; the batch's sub-block table is batch // bps
    b = p // B
    batch = (p - b * B) // 64
    lane = p % 64
    wave, q = batch % 16, batch // 16
    assert (64 * (wave + 16 * q) + lane == p - b * B).all()
    sub = batch // bps
    inside("scatter tab", (sub * pad + ids)[valid], nw * pad)
    inside("scatter lid", 64 * batch + lane, B)
    # bases: ids k0 + tid + 1024 u, u < 8; global loads at present ids only
    inside("scatter segtot", (b // SEG) * n_rows + np.where(valid, ids, 0), nseg * n_rows)
    inside("scatter prefix", b * hist_ld + np.where(valid, ids, 0), nblk * hist_ld)
    # destinations from the decomposition
    v = np.nonzero(valid)[0]
    iv = ids[v]
    cnt = np.bincount(iv, minlength=n_rows)
    seg_off = np.concatenate([[0], np.cumsum(cnt)])[:-1]
    def before(group):  # positions of the same id earlier inside the same group
        key = group * n_rows + iv
        order = np.argsort(key, kind="stable")
        ks = key[order]
        first = np.searchsorted(ks, ks, side="left")
        r = np.empty(v.size, np.int64)
        r[order] = np.arange(v.size) - first
        return r
    seg = b[v] // SEG
    blk = b[v]
    sb = before(np.zeros_like(seg)) - before(seg)                            # earlier segments
    pre = before(seg) - before(blk)                                          # earlier blocks of the segment
    subpre = before(blk) - before(blk * nw + sub[v])                          # earlier sub-blocks of the block
    bat = blk * (B // 64) + batch[v]
    run = before(blk * nw + sub[v]) - before(bat)                             # earlier batches of the sub-block
    rank = before(bat)                                                        # rank in the batch
    assert (rank < 64).all()
    dest = seg_off[iv] + sb + pre + subpre + run + rank
    inside("scatter perm", dest, n_src)
    perm, _ = oi.stable_order(ids, n_rows)
    inv = np.empty(n_src, np.int64)
    inv[perm] = np.arange(perm.size)
    assert (dest == inv[v]).all()


def test_sort_full():
    replay_sort(W.zipf_ids(4096 * 512, 8192, 1.1, 0.05, 3, 0), 8192)


@pytest.mark.parametrize("n_rows", [300, 4000, 16384])
def test_sort_ragged(n_rows):
    rng = np.random.default_rng(n_rows)
    ids = rng.integers(-3, n_rows + 50, 70001)
    ids[100:3000] = n_rows // 2                  # one hot id
    replay_sort(ids, n_rows)


@pytest.mark.parametrize("L", [1, 7, 64, 256, 512, 1024, 65536])
def test_index_add_full(L):
    ids = W.zipf_ids(4096 * 512, 8192, 1.1, 0.05, 3, 0)
    replay_index_add(ids, 8192, 128, L)


def test_index_add_ragged():
    rng = np.random.default_rng(0)
    ids = rng.integers(-3, 1500, 100003)
    ids[:5000] = 17                      # one hot id
    replay_index_add(ids, 1400, 64, 256)  # ids past n_rows are dropped
    replay_index_add(ids, 1400, 64, 7)


@pytest.mark.parametrize("L", [64, 256, 1024])
def test_indexer_dk_full(L):
    x = W.indexer_dk_ids(Q=4096, K=512, n_rows=8192, seed=8)
    Q, K = x.shape
    replay_index_add(x, 8192, 128, L, Q=Q, K=K)
    # ia_coef: wave per query row r < Q, slots 512 c + 8 lane + e < K
    lane = np.arange(64)
    pieces = cdiv(K, 512)
    j = (np.arange(pieces)[:, None, None] * 512 + 8 * lane[None, :, None] + np.arange(8)[None, None, :]).ravel()
    j = j[j < K]
    inside("indexer_dk coef slots", np.array([0, (Q - 1) * K + j.max()]), Q * K)
