"""Host emulation of the index arithmetic of the matrix-core backward (no GPU).

The key-side kernel reads, per (chunk, kv head), a list of rows built by three
passes (per-block counts, a scan, a fill that ranks rows by bitmap popcounts),
and walks it in 32-row tiles, one tile ahead. These tests redo that arithmetic
on the host for the training workload (B=2, T=16384, H=16, K=16) and the main
setting (K=32, a 512-key window), with selections made by the selection rule and
with lists holding entries that do not count, and assert that every record slot
is written exactly once, every list entry a tile (or its prefetch) reads lies
inside the entries written for the current segment, every position and partial
slot is in range, and every dQ partial store lands on a (position, slot) of the
partials or, for a padding row, on the one discard row past them. The constants below mirror the kernel's.
"""
import numpy as np
import pytest

S = 64
LBLK = 256            # positions per block of the list passes
TILE = 32             # rows per key-side tile
KWAVES = 4            # wavefronts per key-side workgroup
LIST_MAX = 64 + 64 * 32
MAX_WINDOW = 16 * S   # larger windows take the vector backward


def lstart(pos, W):
    pos = np.asarray(pos, np.int64)
    return np.where(pos >= W, pos - W + 1, 0) if W > 0 else pos - pos % S


def ncand(pos, W):
    return lstart(pos, W) // S


def counted(idx, n):
    """entry_counts over a [rows, K] list: a candidate above every earlier entry."""
    prev = np.maximum.accumulate(np.concatenate([np.full((idx.shape[0], 1), -1), idx[:, :-1]],
                                                axis=1), axis=1)
    return (idx >= 0) & (idx < n[:, None]) & (idx > prev)


def make_idx(T, K, W, rng, messy):
    pos = np.arange(T)
    n = ncand(pos, W)
    idx = np.full((T, K), -1, np.int32)
    for i in range(T):
        m = min(K, int(n[i]))
        if m:
            idx[i, :m] = np.sort(rng.choice(int(n[i]), size=m, replace=False))
    if messy:  # repeats, swaps, ids past the candidates, negatives
        r = rng.integers(0, T, size=T // 4)
        k = rng.integers(0, K - 1, size=r.size)
        kind = rng.integers(0, 4, size=r.size)
        for rr, kk, kd in zip(r, k, kind):
            if kd == 0:
                idx[rr, kk + 1] = idx[rr, kk]
            elif kd == 1:
                idx[rr, [kk, kk + 1]] = idx[rr, [kk + 1, kk]]
            elif kd == 2:
                idx[rr, kk] = n[rr] + 1
            else:
                idx[rr, kk] = -7
    return idx, n


def emulate_head(idx, n, T, K, W, NC):
    """One (b, h): count/scan/fill, then the key-side walk of every chunk."""
    NL = W // S + 1 if W > 0 else 1
    ok = counted(idx, n)
    nblk = (T + LBLK - 1) // LBLK
    rows, ks = np.nonzero(ok)
    cs = idx[rows, ks]
    # k_sel_count + k_sel_scan: offsets in (chunk, block) order
    cnt = np.zeros((NC, nblk), np.int64)
    np.add.at(cnt, (cs, rows // LBLK), 1)
    off = np.concatenate([[0], np.cumsum(cnt.reshape(-1))])[:-1].reshape(NC, nblk)
    total = int(cnt.sum())
    lst = off[:, 0]
    llen = np.append(lst[1:], total) - lst
    # k_sel_fill: rank of a row among the block's rows that selected the chunk
    srec_pos = np.full(total, -1, np.int64)
    srec_slot = np.full(total, -1, np.int64)
    written = np.zeros(total, np.int64)
    order = np.lexsort((rows, cs))
    rr, kk, cc = rows[order], ks[order], cs[order]
    first = np.ones(rr.size, bool)
    first[1:] = (cc[1:] != cc[:-1]) | (rr[1:] // LBLK != rr[:-1] // LBLK)
    grp = np.cumsum(first) - 1
    start = np.flatnonzero(first)
    rank = np.arange(rr.size) - start[grp]
    dst = off[cc, rr // LBLK] + rank
    assert dst.min() >= 0 and dst.max() < total
    np.add.at(written, dst, 1)
    assert np.all(written == 1), "a record slot written twice or never"
    srec_pos[dst] = rr
    srec_slot[dst] = kk
    # every record of chunk c lies in [lst[c], lst[c] + llen[c]) and names a row that
    # selected c in the given slot
    assert np.all((dst >= lst[cc]) & (dst < lst[cc] + llen[cc]))
    assert np.all(idx[srec_pos, srec_slot] == np.repeat(np.arange(NC), llen))
    # key-side walk: list segments and tiles, with the next tile prefetched
    span = S + W - 1 if W > 0 else S
    for c in range(NC):
        key0 = c * S
        LN = int(llen[c])
        nown = min(span, T - key0)
        nown_pad = (nown + TILE - 1) // TILE * TILE
        kseg = LIST_MAX - nown_pad
        assert kseg > 0
        s0 = 0
        while True:
            base = nown_pad if s0 == 0 else 0
            ns = min(kseg, LN - s0)
            nn = base + ns
            assert 0 <= nn <= LIST_MAX
            seg_pos = np.empty(nn, np.int64)
            seg_slot = np.empty(nn, np.int64)
            e = np.arange(base)
            p = key0 + np.minimum(e, nown - 1)
            seg_pos[:base] = p
            seg_slot[:base] = np.where(e < nown, K + (c - lstart(p, W) // S), -1)
            src = lst[c] + s0 + np.arange(ns)
            seg_pos[base:] = srec_pos[src]
            seg_slot[base:] = srec_slot[src]
            assert np.all((seg_pos >= 0) & (seg_pos < T))
            assert np.all((seg_slot >= -1) & (seg_slot < K + NL))
            assert np.all(seg_slot[:nown] >= K) if s0 == 0 else True
            for w in range(KWAVES):
                e0 = TILE * w
                while e0 < nn:
                    e1 = e0 + TILE * KWAVES
                    for ep in (e0, e1 if e1 < nn else e0):  # the tile and its prefetch
                        nr = min(TILE, nn - ep)
                        lanes = np.arange(64)
                        reads = [ep + np.minimum(8 * i + (lanes >> 3), nr - 1) for i in range(4)]
                        reads += [ep + np.minimum(16 * hf + (lanes & 15), nr - 1) for hf in range(2)]
                        for rd in reads:
                            assert rd.min() >= 0 and rd.max() < nn
                    # the tile's dQ partial stores: a row that counts writes its
                    # (position, slot), a padding row the discard row past them
                    nr = min(TILE, nn - e0)
                    for hf in range(2):
                        lr = 16 * hf + (np.arange(64) & 15)
                        e = e0 + np.minimum(lr, nr - 1)
                        slot = seg_slot[e]
                        rpos = np.where((lr < nr) & (slot >= 0), seg_pos[e], -1)
                        dst = np.where(rpos >= 0, rpos * (K + NL) + slot, T * (K + NL))
                        assert dst.min() >= 0 and dst.max() <= T * (K + NL)
                        assert np.all((rpos < 0) | (slot < K + NL))
                    e0 = e1
            if s0 + kseg >= LN:
                break
            s0 += kseg


@pytest.mark.parametrize("K,W,messy", [(16, 0, False), (16, 0, True), (32, 512, False),
                                       (32, 512, True), (64, 1024, True)])
def test_backward_list_and_tile_indices(K, W, messy):
    assert W <= MAX_WINDOW
    T = 16384
    NC = T // S
    rng = np.random.default_rng(K + W + messy)
    for head in range(2):  # two (b, h) lists per case keep the run short
        idx, n = make_idx(T, K, W, rng, messy)
        emulate_head(idx, n, T, K, W, NC)
