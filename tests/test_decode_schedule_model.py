"""CPU model of the decode work split (host-side reasoning behind the device
schedule): the key blocks of all (sequence, KV head, head chunk) pairs are cut
into equal contiguous worker ranges; each worker finds its first unit by
scanning the per-sequence block counts; every piece is written to slot
(piece index + worker index); the merge pass finds exactly the workers that
wrote each piece.  Checked exhaustively on random small problems, including
more workers than units and sequences of length 0."""
import random


def _blocks(L):
    return (L + 63) // 64


def _locate(nb, t):
    """Sequence b with prefix[b] <= t < prefix[b+1], and prefix[b]."""
    run = 0
    for b, n in enumerate(nb):
        if n > 0 and run <= t < run + n:
            return b, run
        run += n
    return len(nb), run


def _check(lens, hkhc, P):
    nb = [_blocks(L) for L in lens]
    B = len(nb)
    W = sum(nb) * hkhc
    written = {}
    covered = []
    for w in range(P):
        ub, ue = W * w // P, W * (w + 1) // P
        if ub >= ue:
            continue
        b, before = _locate(nb, ub // hkhc)
        rem = ub - before * hkhc
        ql, j = divmod(rem, nb[b])
        for _ in range(ue - ub):
            covered.append((b, ql, j))
            slot = b * hkhc + ql + w
            assert written.setdefault(slot, (b, ql)) == (b, ql), "two pieces share a slot"
            j += 1
            if j == nb[b]:
                j, ql = 0, ql + 1
                if ql == hkhc:
                    ql, b = 0, b + 1
                    while b < B and nb[b] == 0:
                        b += 1
    assert covered == [(b, ql, j) for b in range(B) for ql in range(hkhc) for j in range(nb[b])]
    pre = [0]
    for n in nb:
        pre.append(pre[-1] + n)
    for b in range(B):
        for ql in range(hkhc):
            if nb[b] == 0:
                continue
            u0 = pre[b] * hkhc + ql * nb[b]
            u1 = u0 + nb[b]
            w0, w1 = ((u0 + 1) * P - 1) // W, (u1 * P - 1) // W
            found = {w for w in range(w0, w1 + 1) if W * w // P < W * (w + 1) // P}
            want = {s - (b * hkhc + ql) for s, v in written.items() if v == (b, ql)}
            assert found == want


def test_work_split_covers_every_block_once_and_slots_are_unique():
    rng = random.Random(0)
    n = 0
    while n < 1500:
        B = rng.randint(1, 7)
        lens = [rng.choice([0, 1, 63, 64, 65, 130, rng.randint(0, 900)]) for _ in range(B)]
        if sum(lens) == 0:
            continue
        _check(lens, rng.choice([1, 2, 3, 8]), rng.choice([1, 2, 3, 5, 7, 10, 33, 100, 1024]))
        n += 1
