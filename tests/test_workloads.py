"""The seeded input generators: determinism and the structure each config promises."""
import numpy as np

from workloads import gen


def test_decode_generation_is_deterministic():
    a = gen.make_decode_case(name="a", seed=77, B=3, Hq=4, Hk=2, D=16, q_dtype="bf16",
                             kv_dtype="e4m3fn", len_range=(1, 200))
    b = gen.make_decode_case(name="b", seed=77, B=3, Hq=4, Hk=2, D=16, q_dtype="bf16",
                             kv_dtype="e4m3fn", len_range=(1, 200))
    for x, y in [(a.q, b.q), (a.k_pool, b.k_pool), (a.v_pool, b.v_pool),
                 (a.block_table, b.block_table), (a.seq_lens, b.seq_lens)]:
        np.testing.assert_array_equal(x, y)
    assert a.k_scale == b.k_scale and a.v_scale == b.v_scale


def test_tiny_fp32_config_structure():
    c = gen.decode_tiny_fp32()
    assert c.q.shape == (2, 8, 64) and c.k_pool.shape == (6, 4, 64, 64)
    assert list(c.seq_lens) == [100, 37] and c.block_table.shape == (2, 2)
    assert len(set(c.block_table.ravel().tolist())) == 4          # injective
    used = {int(c.block_table[0, 0]), int(c.block_table[0, 1]), int(c.block_table[1, 0])}
    for blk in range(6):
        nan_rows = np.isnan(c.k_pool[blk, 0, :, 0])
        if blk not in used:
            assert nan_rows.all()                                  # incl. block_table[1, 1]
    assert np.isnan(c.k_pool[c.block_table[0, 1], :, 36:]).all()
    assert not np.isnan(c.k_pool[c.block_table[0, 1], :, :36]).any()
    assert np.isnan(c.v_pool[c.block_table[1, 0], :, 37:]).all()
    assert not np.isnan(c.v_pool[c.block_table[1, 0], :, :37]).any()


def test_gqa_decode_pool_is_exactly_the_needed_blocks():
    c = gen.make_decode_case(name="t", seed=1002, B=8, Hq=32, Hk=8, D=128, q_dtype="bf16",
                             kv_dtype="bf16", len_range=(1024, 4096))
    need = (c.seq_lens + 63) // 64
    assert c.NB == need.sum()
    ids = np.concatenate([c.block_table[b, :need[b]] for b in range(c.B)])
    assert sorted(ids.tolist()) == list(range(c.NB))               # a permutation of the pool
    for b in range(c.B):
        assert np.all(c.block_table[b, need[b]:] == -1)
    assert np.all((c.seq_lens >= 1024) & (c.seq_lens <= 4096))


def test_fp8_scales_are_amax_over_448():
    c = gen.make_decode_case(name="t", seed=3, B=2, Hq=8, Hk=1, D=32, q_dtype="bf16",
                             kv_dtype="e4m3fn", seq_lens=[64, 64])
    # the largest code magnitude is 448 (0x7E) exactly: amax / scale == 448 before rounding
    mags = c.k_pool & 0x7F
    assert mags[mags != 0x7F].max() == 0x7E


def test_blocksparse_mask_structure():
    p = gen.make_prefill_case(name="t", seed=1005, seq_lens=[1024, 1024], Hq=4, Hk=1,
                              D_qk=16, D_rope=0, D_v=16, mask_density=0.25)
    m = p.block_mask
    nb = m.shape[1]
    assert m.shape == (2, nb, nb) and nb == 16
    assert np.all(m[:, np.arange(nb), np.arange(nb)] == 1)
    assert np.all(m[:, :, 0] == 1)
    assert np.all(np.triu(m, 1) == 0)
    off = np.tril(np.ones((nb, nb), bool), -1)
    off[:, 0] = False
    frac = m[:, off].mean()
    assert 0.1 < frac < 0.4


def test_ragged_prefill_offsets():
    p = gen.prefill_mla_bf16()
    assert p.q.shape == (6584, 16, 192) and p.k.shape == (6584, 16, 128)
    assert p.k_rope.shape == (6584, 1, 64) and p.v.shape == (6584, 16, 128)


def test_chunk_case_structure():
    """Prefix rows filled, every other pool row NaN; kv_len = prefix + chunk;
    the table covers ceil(kv_len / 64) distinct blocks; deterministic."""
    c = gen.make_chunk_case(name="t", seed=7, prefix_lens=[0, 63, 130], q_lens=[5, 1, 64], Hq=4, Hk=2)
    assert c.kv_lens.tolist() == [5, 64, 194] and c.cu_seqlens_q.tolist() == [0, 5, 6, 70]
    assert c.k_pool.shape == (1 + 1 + 4 + 2, 2, 64, 128)
    used = [int(x) for row, L in zip(c.block_table, c.kv_lens) for x in row[: (L + 63) // 64]]
    assert len(set(used)) == len(used) == 6 and all(x == -1 for x in c.block_table[0, 1:])
    finite = np.zeros(c.k_pool.shape[:1] + (64,), bool)
    for b, p in enumerate([0, 63, 130]):
        for t in range(p):
            finite[c.block_table[b, t // 64], t % 64] = True
    rows = c.k_pool.transpose(0, 2, 1, 3)                      # [NB, 64, Hk, D]
    assert np.all(rows[~finite] == gen.BF16_NAN) and not np.any(rows[finite] == gen.BF16_NAN)
    c2 = gen.make_chunk_case(name="t", seed=7, prefix_lens=[0, 63, 130], q_lens=[5, 1, 64], Hq=4, Hk=2)
    assert np.array_equal(c.q, c2.q) and np.array_equal(c.k_pool, c2.k_pool)
    # visible pairs: query i of chunk b sees prefix_b + i + 1 keys
    assert c.visible_pairs() == sum(p * q + q * (q + 1) // 2 for p, q in ((0, 5), (63, 1), (130, 64)))
