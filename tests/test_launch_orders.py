"""CPU emulation of two index constructions of the HIP path (no GPU).

1. The prefill attention's claim list: per workgroup, the selected chunks of at
   least 33 rows first, then the others, each group in ascending chunk order,
   placed from one exclusive scan of a packed (heavy << 16 | light) count per
   chunk; the wavefronts claim the list in order.
2. The backward key side's launch order: the (chunk, kv head, b) workgroups in
   buckets of log2 of their 32-row tiles, the largest bucket first, each bucket's
   places handed out by a counter.

Both must be permutations (every chunk or workgroup exactly once), with the
stated order; the results of the kernels do not depend on the order, so these
checks cover what the order could break: a chunk or workgroup lost or doubled.
"""
import numpy as np
import pytest

HEAVY_ROWS = 33   # k_attend_mfma.hip: kHeavyRows
CHUNK = 64        # own rows of a chunk per head in the key side


def claim_list(cnt):
    """cnt[c] = rows of the workgroup that selected chunk c (c < ncr)."""
    packed = np.where(cnt >= HEAVY_ROWS, 1 << 16, np.where(cnt > 0, 1, 0)).astype(np.int64)
    excl = np.concatenate([[0], np.cumsum(packed)[:-1]])
    tot = int(packed.sum())
    nheavy, nnz = tot >> 16, (tot >> 16) + (tot & 0xFFFF)
    cur = np.full(nnz, -1, dtype=np.int64)
    for c in range(len(cnt)):
        x = int(excl[c])
        if cnt[c] >= HEAVY_ROWS:
            assert cur[x >> 16] == -1
            cur[x >> 16] = c
        elif cnt[c] > 0:
            assert cur[nheavy + (x & 0xFFFF)] == -1
            cur[nheavy + (x & 0xFFFF)] = c
    return cur, nheavy


@pytest.mark.parametrize("seed", range(6))
def test_attention_claim_list(seed):
    rng = np.random.default_rng(seed)
    ncr = int(rng.integers(1, 1025))
    cnt = rng.integers(0, 40, ncr)                      # light chunks and empty ones
    heavy = rng.random(ncr) < 0.05
    cnt[heavy] = rng.integers(HEAVY_ROWS, 257, int(heavy.sum()))
    cur, nheavy = claim_list(cnt)
    sel = np.nonzero(cnt > 0)[0]
    assert sorted(cur.tolist()) == sel.tolist()        # every selected chunk once
    assert all(cnt[cur[:nheavy]] >= HEAVY_ROWS) and all(cnt[cur[nheavy:]] < HEAVY_ROWS)
    assert np.all(np.diff(cur[:nheavy]) > 0) and np.all(np.diff(cur[nheavy:]) > 0)


def bwd_order(llen, B, Hkv, G, NC):
    """llen[b, h, c]: selecting rows of (b, head h, chunk c); returns order[i] = L."""
    n = NC * Hkv * B

    def bucket(L):
        g, b, c = L % Hkv, (L // Hkv) % B, L // (Hkv * B)
        rows = sum(CHUNK + int(llen[b, g * G + hh, c]) for hh in range(G))
        tiles = max((rows + 31) // 32, 1)
        return min(15, tiles.bit_length() - 1)

    bk = [bucket(L) for L in range(n)]
    hist = np.bincount(bk, minlength=16)
    fill = np.zeros(16, dtype=np.int64)
    order = np.full(n, -1, dtype=np.int64)
    for L in np.random.default_rng(0).permutation(n):  # the atomics' order is free
        start = int(hist[bk[L] + 1:].sum())
        pos = start + int(fill[bk[L]])
        fill[bk[L]] += 1
        assert order[pos] == -1
        order[pos] = L
    return order, bk


@pytest.mark.parametrize("B,Hkv,G,NC", [(2, 16, 1, 256), (1, 8, 4, 64), (2, 2, 2, 33)])
def test_backward_launch_order(B, Hkv, G, NC):
    rng = np.random.default_rng(B * 100 + NC)
    llen = rng.integers(0, 1200, (B, Hkv * G, NC))
    llen[rng.random(llen.shape) < 0.01] = 8448          # a few chunks most rows selected
    order, bk = bwd_order(llen, B, Hkv, G, NC)
    assert sorted(order.tolist()) == list(range(NC * Hkv * B))
    b = np.array(bk)[order]
    assert np.all(np.diff(b) <= 0)                      # largest tile bucket first
