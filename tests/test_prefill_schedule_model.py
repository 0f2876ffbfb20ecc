"""Host model of how the prefill kernel maps its grid to work (no GPU).

Workgroup i of the one-dimensional grid takes head slot x = i % NH (NH = Hq /
hpw workgroups per item: one head with hpw = 1, a pair of heads of one KV
group with hpw = 2), key-axis split sp = (i // NH) % S, and the
(i // NH // S)-th existing (sequence, query tile) item, items ranked deepest
query tile first, then by sequence (for up to 64 sequences a wave ranks them
with one ballot per depth, and the grid holds only as many items as the rows
can fill, (T + B (QT - 1)) / QT; past 64 the order is plain).  A paged grid
of more than one round of workgroups (up to 64 sequences) ranks its items
instead by the keys the tile's last row sees, off + min(Lq, (qt + 1) QT) with
off the cached keys before the chunk, most first, ties by sequence; a wave
finds the item of a rank by a binary search over that key count.  A query tile has
QT = 128 / hpw rows; split sp takes key tiles [nkt sp / S, nkt (sp+1) / S)
of the nkt tiles the tile needs.  Rows of a sequence past the plan's
capacity are cleared by split 0 of the sequence's last query tile.

This model restates that mapping and checks, on random problems:
  * every (sequence, head, query row) within the capacity is computed by
    exactly one workgroup per split, and the splits' key ranges partition
    the tile's key tiles;
  * every row past the capacity is cleared exactly once, by a workgroup of
    its own head, and never also computed;
  * the block-mask reads stay inside the sequence's [nb, nb] slice;
  * the kernel's binary-search inversion of the ranking gives the item
    that sorting the items by key count gives, for every rank;
  * the real items precede the empty tail of the grid (ranked path), and
  * the heads of one KV group share an XCD (workgroup i runs on XCD i % 8)
    whenever the group fits in one XCD's share of the heads."""
import numpy as np
import pytest


def item_tiles(Lq, max_len, q_tiles, QT):
    return 0 if Lq <= 0 else q_tiles if Lq > max_len else -(-Lq // QT)


def rank(lens, max_len, q_tiles, QT, item, offs=None, by_keys=False):
    """(b, qt) of grid item `item`, or None (the workgroup returns at once)."""
    B = len(lens)
    nq = [item_tiles(L, max_len, q_tiles, QT) for L in lens]
    if B <= 64 and by_keys:
        offs = offs or [0] * B
        items = sorted(((offs[b] + min(lens[b], (qt + 1) * QT), b, qt) for b in range(B) for qt in range(nq[b])),
                       key=lambda e: (-e[0], e[1]))
        return (items[item][1], items[item][2]) if item < len(items) else None
    if B <= 64:
        before = 0
        for t in range(q_tiles - 1, -1, -1):
            members = [b for b in range(B) if nq[b] > t]      # ballot(nq > t), lane order
            if item < before + len(members):
                return members[item - before], t
            before += len(members)
        return None
    b, qt = item % B, q_tiles - 1 - item // B
    return (b, qt) if qt < item_tiles(lens[b], max_len, q_tiles, QT) else None


def rank_by_search(lens, max_len, q_tiles, QT, item, offs):
    """The kernel's steps for up to 64 sequences: lane b holds lq, nq and the
    key offset; deeper(v) counts its items whose key count exceeds v; a
    binary search finds the key count of the rank, a ballot the sequence."""
    B = len(lens)
    qsh = QT.bit_length() - 1
    nq = [item_tiles(L, max_len, q_tiles, QT) for L in lens]
    koff = [max(0, o) for o in offs]

    def deeper(b, v):
        y = v - koff[b]
        if nq[b] == 0 or lens[b] <= y:
            return 0
        return nq[b] if y < 0 else max(0, nq[b] - (y >> qsh))

    if item >= sum(nq):
        return None
    lo, hi = -1, max(koff[b] + lens[b] for b in range(B))
    while hi - lo > 1:
        mid = lo + ((hi - lo) >> 1)
        if sum(deeper(b, mid) for b in range(B)) <= item:
            hi = mid
        else:
            lo = mid
    above = sum(deeper(b, hi) for b in range(B))
    members = [b for b in range(B) if deeper(b, hi - 1) > deeper(b, hi)]   # ballot, lane order
    b = members[item - above]
    return b, nq[b] - deeper(b, hi - 1)


def rank_parallel(lens, max_len, q_tiles, QT, item):
    """The kernel's parallel form of the query-tile ranking (used when
    q_tiles > 32 and B ceil(q_tiles / 64) < q_tiles): C(t) = sum_b max(0, nq_b - t) items have a
    tile index >= t; the item's tile index is one less than the number of t
    with C(t) > item; a ballot over nq_b > qt then picks the sequence."""
    B = len(lens)
    nq = [item_tiles(L, max_len, q_tiles, QT) for L in lens]
    above = sum(1 for t in range(q_tiles) if sum(max(0, n - t) for n in nq) > item)
    if above == 0:
        return None
    qt = above - 1
    before = sum(max(0, n - above) for n in nq)
    members = [b for b in range(B) if nq[b] > qt]
    return members[item - before], qt


def head_of(x, NH):
    hpx = NH >> 3
    return x if NH & 7 else (x & 7) * hpx + (x >> 3)


def simulate(lens, max_len, Hq, Hk, hpw, S, nb=None):
    QT = 128 // hpw
    NH = Hq // hpw
    ratio = Hq // Hk
    q_tiles = max(1 if lens else 0, -(-max_len // QT))
    items = len(lens) * q_tiles
    if len(lens) <= 64:   # the launch holds no more items than the rows can fill
        T = sum(max(L, 0) for L in lens)
        items = min(items, max(1 if lens else 0, (T + len(lens) * (QT - 1)) // QT))
    grid = NH * items * S
    computed = {}      # (b, h, row) -> list of (sp, key-tile range)
    cleared = {}       # (b, h, row) -> count
    mask_rows = []     # (b, mask row index) read
    served_items = []
    for i in range(grid):
        x, sp, item = i % NH, (i // NH) % S, i // NH // S
        r = rank(lens, max_len, q_tiles, QT, item)
        if sp == 0 and x == 0:
            served_items.append(r)
        if r is None:
            continue
        b, qt = r
        hx = head_of(x, NH)
        heads = [hx] if hpw == 1 else [2 * hx, 2 * hx + 1]
        assert len({h // ratio for h in heads}) == 1        # a pair shares its KV head
        Lq = lens[b]
        L = min(Lq, max_len)
        nqb = item_tiles(Lq, max_len, q_tiles, QT)
        if Lq > L and sp == 0 and qt == nqb - 1:
            for h in heads:
                for row in range(L, Lq):
                    cleared[(b, h, row)] = cleared.get((b, h, row), 0) + 1
        q0 = qt * QT
        if q0 >= L:
            continue
        nkt = -(-min(L, q0 + QT) // 64)
        kt0, kt1 = nkt * sp // S, nkt * (sp + 1) // S
        for wv in range(4):
            wslot = (wv & 1) if hpw == 2 else wv
            h = 2 * hx + (wv >> 1) if hpw == 2 else hx
            r0 = q0 + 32 * wslot
            wave_rows = r0 < L
            qb0, qb1, wqb = q0 >> 6, min((q0 + QT - 1) >> 6, (L - 1) >> 6), r0 >> 6
            if nb is not None:                             # rows of the mask the wave reads
                mask_rows += [(b, qb0), (b, qb1)] + ([(b, wqb)] if wave_rows else [])
            for row in range(r0, min(r0 + 32, L)):
                computed.setdefault((b, h, row), []).append((sp, kt0, kt1, nkt))
    return computed, cleared, mask_rows, served_items


CASES = []
rng0 = np.random.default_rng(7)
for k in range(36):
    B = int(rng0.choice([1, 2, 5, 63, 64, 65, 90]))
    hpw = int(rng0.choice([1, 2]))
    Hk = int(rng0.choice([1, 2, 4]))
    ratio = int(rng0.choice([2, 4])) if hpw == 2 else int(rng0.choice([1, 2, 4]))
    CASES.append((k, B, hpw, Hk, Hk * ratio, int(rng0.choice([1, 2, 3, 4]))))


@pytest.mark.parametrize("seed,B,hpw,Hk,Hq,S", CASES)
def test_grid_covers_every_row_once(seed, B, hpw, Hk, Hq, S):
    rng = np.random.default_rng(seed)
    lens = rng.integers(0, 700, size=B).tolist()
    if seed % 4 == 0:
        lens[0] = 0
    cap = int(rng.choice([max(lens + [1]), 256, 129, 64, 0]))   # capacities below the longest sequence too
    nb = max(1, -(-cap // 64))
    computed, cleared, mask_rows, served = simulate(lens, cap, Hq, Hk, hpw, S, nb=nb)
    for b, Lq in enumerate(lens):
        L = min(Lq, cap)
        for h in range(Hq):
            for row in range(max(Lq, 0)):
                key = (b, h, row)
                if row < L:
                    parts = computed.get(key, [])
                    assert sorted(p[0] for p in parts) == list(range(S)), key
                    nkt = parts[0][3]
                    tiles = sorted(t for _, a, e, _ in parts for t in range(a, e))
                    assert tiles == list(range(nkt)) and nkt * 64 >= row + 1, key
                    assert key not in cleared
                else:
                    assert cleared.get(key) == 1 and key not in computed, key
    assert len(computed) == sum(min(L, cap) for L in lens) * Hq
    assert all(0 <= r < nb for _, r in mask_rows)
    if B <= 64:
        k = sum(1 for s in served if s is not None)
        assert all(s is not None for s in served[:k]) and all(s is None for s in served[k:])
        depths = [t for _, t in served[:k]]
        assert depths == sorted(depths, reverse=True)


@pytest.mark.parametrize("Hq,Hk,hpw", [(32, 8, 1), (32, 8, 2), (64, 8, 1), (16, 2, 2), (128, 16, 1)])
def test_heads_of_one_kv_group_share_an_xcd(Hq, Hk, hpw):
    """With NH a multiple of 8, workgroup i runs on XCD i % 8 = x % 8, and the
    slots x with one x % 8 take NH / 8 consecutive heads (or head pairs)."""
    NH = Hq // hpw
    ratio = Hq // Hk
    xcd_of_group = {}
    for x in range(NH):
        hx = head_of(x, NH)
        heads = [hx] if hpw == 1 else [2 * hx, 2 * hx + 1]
        for h in heads:
            xcd_of_group.setdefault(h // ratio, set()).add(x % 8)
    if (NH // 8) % max(1, ratio // hpw) == 0:
        assert all(len(s) == 1 for s in xcd_of_group.values())


@pytest.mark.parametrize("seed", range(24))
def test_kernel_rank_inversion_matches_the_sorted_order(seed):
    """The key-count ranking: the binary search and ballot give, rank for
    rank, the items sorted by key count (most first, ties by sequence), and
    the ranks past the last item give none."""
    rng = np.random.default_rng(100 + seed)
    B = int(rng.integers(1, 65))
    QT = int(rng.choice([64, 128]))
    lens = [int(x) for x in rng.integers(0, 700, size=B)]
    lens[int(rng.integers(0, B))] = 0
    offs = [int(x) for x in rng.integers(0, 5000, size=B)] if seed % 2 else [0] * B
    max_len = int(rng.choice([max(lens) + 1, max(1, max(lens) // 2)]))  # some sequences past the capacity
    q_tiles = max(1, -(-max_len // QT))
    total = sum(item_tiles(L, max_len, q_tiles, QT) for L in lens)
    got = [rank_by_search(lens, max_len, q_tiles, QT, i, offs) for i in range(total + 3)]
    want = [rank(lens, max_len, q_tiles, QT, i, offs, by_keys=True) for i in range(total + 3)]
    assert got == want
    assert got[total:] == [None] * 3 and len(set(got[:total])) == total
    keys = [offs[b] + min(lens[b], (qt + 1) * QT) for b, qt in got[:total]]
    assert keys == sorted(keys, reverse=True)


@pytest.mark.parametrize("seed", range(24))
def test_parallel_tile_ranking_matches_the_tile_walk(seed):
    """The parallel query-tile ranking gives, rank for rank, the item of the
    walk over tile indices (deepest first, then by sequence)."""
    rng = np.random.default_rng(200 + seed)
    B = int(rng.integers(1, 65))
    QT = int(rng.choice([64, 128]))
    lens = [int(x) for x in rng.integers(0, 9000 if seed % 3 else 700, size=B)]
    lens[int(rng.integers(0, B))] = 0
    max_len = int(rng.choice([max(lens) + 1, max(1, max(lens) // 2)]))
    q_tiles = max(1, -(-max_len // QT))
    total = sum(item_tiles(L, max_len, q_tiles, QT) for L in lens)
    got = [rank_parallel(lens, max_len, q_tiles, QT, i) for i in range(total + 3)]
    want = [rank(lens, max_len, q_tiles, QT, i) for i in range(total + 3)]
    assert got == want
