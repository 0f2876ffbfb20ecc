"""Host model of how the prefill kernel ranks its work items (no GPU).

Workgroup i of the one-dimensional grid serves query head i % Hq and the
(i // Hq)-th existing (sequence, 128-row query tile) pair, pairs ranked
deepest query tile first, then by sequence (for up to 64 sequences a wave
ranks them with one ballot per depth).  This model restates that ranking and
checks that every pair is served exactly once, that the grid covers them
all, and that the tail past the last pair is empty."""
import numpy as np
import pytest


def kernel_rank(lens, max_len, pair):
    """(b, qt) of grid pair `pair`, or None past the last real pair."""
    B = len(lens)
    q_tiles = -(-max_len // 128)
    if B <= 64:
        nq = [(min(L, max_len) + 127) // 128 for L in lens]
        before = 0
        for t in range(q_tiles - 1, -1, -1):
            members = [b for b in range(B) if nq[b] > t]     # ballot(nq > t), lane order
            if pair < before + len(members):
                return members[pair - before], t
            before += len(members)
        return None
    b, qt = pair % B, q_tiles - 1 - pair // B
    return (b, qt) if qt * 128 < min(lens[b], max_len) else None


@pytest.mark.parametrize("seed", range(40))
def test_every_query_tile_served_once(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.choice([1, 2, 7, 63, 64, 65, 100]))
    lens = rng.integers(0, 3000, size=B).tolist()
    if seed % 5 == 0:
        lens[0] = 0
    max_len = max(lens + [1])
    q_tiles = -(-max_len // 128)
    served = [kernel_rank(lens, max_len, p) for p in range(B * q_tiles)]
    real = [s for s in served if s is not None]
    want = {(b, t) for b, L in enumerate(lens) for t in range(-(-L // 128))}
    assert len(real) == len(set(real)) == len(want) and set(real) == want
    if B <= 64:
        # dense: real pairs first, then only empty slots; deepest first
        k = len(real)
        assert all(s is not None for s in served[:k]) and all(s is None for s in served[k:])
        depths = [t for _, t in real]
        assert depths == sorted(depths, reverse=True)
