"""Pins of the chunked-prefill and append parts of the oracle (CPU only).

Chunked prefill (FlashMLA tensor-shape reference, section 4 and its "Prefill to
Cache Mapping"; MATE msa_interface _normalize_qo_offset / _resolve_seqused_k):
a sequence holds kv_len keys in the paged cache, the last q_len being the
chunk's own tokens, and query i sees key j iff j <= kv_len - q_len + i.

Each pin checks the oracle against something other than itself: pure-Python
brute force on the unpaged tensors, a torch SDPA with an explicit offset mask,
reductions to the ragged-prefill and decode definitions, and the
split-a-sequence-into-chunks identity.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import attention as O
from oracle import bruteforce as BF


def _pool_case(seed, kv_lens, q_lens, Hq, Hk, D, extra_blocks=2):
    """Random logical K/V per sequence, scattered into a NaN pool through a
    shuffled block table (token t -> block table[b][t // 64], row t % 64)."""
    rng = np.random.default_rng(seed)
    B = len(kv_lens)
    nblk = max(1, max((L + 63) // 64 for L in kv_lens))
    NB = B * nblk + extra_blocks
    table = rng.permutation(NB)[: B * nblk].reshape(B, nblk).astype(np.int32)
    K = [rng.standard_normal((L, Hk, D)) for L in kv_lens]
    V = [rng.standard_normal((L, Hk, D)) for L in kv_lens]
    kp = np.full((NB, Hk, 64, D), np.nan)
    vp = np.full((NB, Hk, 64, D), np.nan)
    for b, L in enumerate(kv_lens):
        for t in range(L):
            kp[table[b][t // 64], :, t % 64] = K[b][t]
            vp[table[b][t // 64], :, t % 64] = V[b][t]
    cu = O.cu_seqlens_from_lengths(q_lens)
    q = rng.standard_normal((int(cu[-1]), Hq, D))
    return q, K, V, kp, vp, table, cu, np.asarray(kv_lens, np.int32)


def _cat(lists):
    return np.concatenate([np.array(x) for x in lists]) if lists else np.zeros((0,))


@pytest.mark.parametrize("Hq,Hk", [(4, 4), (4, 1), (6, 2)])
def test_chunk_prefill_matches_bruteforce(Hq, Hk):
    kv_lens, q_lens = [70, 5, 130, 64], [6, 5, 64, 1]     # prefixes 64, 0, 66, 63
    q, K, V, kp, vp, table, cu, kvl = _pool_case(41, kv_lens, q_lens, Hq, Hk, 8)
    out, lse = O.chunk_prefill(q, kp, vp, table, cu, kvl, 0.35)
    qs = [q[cu[b]:cu[b + 1]] for b in range(len(q_lens))]
    bo, bl = BF.chunk_prefill(qs, K, V, [kv_lens[b] - q_lens[b] for b in range(len(q_lens))], 0.35)
    np.testing.assert_allclose(out, _cat(bo), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, _cat(bl), rtol=0, atol=1e-12)


def test_chunk_prefill_matches_sdpa_with_offset_mask():
    """torch fp64 SDPA over the unpaged keys with the boolean mask j <= o + i."""
    kv_lens, q_lens = [200, 97], [77, 97]
    Hq, Hk, D, scale = 8, 2, 16, 0.25
    q, K, V, kp, vp, table, cu, kvl = _pool_case(42, kv_lens, q_lens, Hq, Hk, D)
    out, lse = O.chunk_prefill(q, kp, vp, table, cu, kvl, scale)
    for b in range(2):
        n, Lk = q_lens[b], kv_lens[b]
        off = Lk - n
        qb = torch.from_numpy(q[cu[b]:cu[b + 1]]).permute(1, 0, 2)              # [Hq, n, D]
        kb = torch.from_numpy(K[b]).permute(1, 0, 2).repeat_interleave(Hq // Hk, 0)
        vb = torch.from_numpy(V[b]).permute(1, 0, 2).repeat_interleave(Hq // Hk, 0)
        m = torch.arange(Lk)[None, :] <= (off + torch.arange(n))[:, None]
        ref = F.scaled_dot_product_attention(qb, kb, vb, attn_mask=m, scale=scale).permute(1, 0, 2)
        np.testing.assert_allclose(out[cu[b]:cu[b + 1]], ref.numpy(), rtol=0, atol=1e-10)
        s = scale * torch.matmul(qb, kb.transpose(-1, -2).contiguous()).masked_fill(~m, float("-inf"))
        np.testing.assert_allclose(lse[cu[b]:cu[b + 1]], torch.logsumexp(s, -1).T.numpy(), rtol=0, atol=1e-10)


def test_chunk_with_empty_prefix_equals_ragged_prefill():
    """kv_len == q_len: the chunk is a whole sequence, so the result is the
    causal ragged prefill of the same logical tensors."""
    lens = [1, 64, 100]
    q, K, V, kp, vp, table, cu, kvl = _pool_case(43, lens, lens, 4, 2, 12)
    out, lse = O.chunk_prefill(q, kp, vp, table, cu, kvl, 0.3)
    k = np.concatenate(K)
    v = np.concatenate(V)
    ro, rl = O.ragged_prefill(q, k, v, cu, 0.3)
    np.testing.assert_allclose(out, ro, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, rl, rtol=0, atol=1e-12)


def test_one_token_chunk_equals_decode():
    """q_len == 1: the single query is the newest token and sees every key,
    which is the decode definition."""
    kv_lens = [1, 65, 130]
    q, K, V, kp, vp, table, cu, kvl = _pool_case(44, kv_lens, [1, 1, 1], 8, 2, 16)
    out, lse = O.chunk_prefill(q, kp, vp, table, cu, kvl, 0.2)
    do, dl = O.paged_decode(q, kp, vp, table, kvl, 0.2)
    np.testing.assert_allclose(out, do, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, dl, rtol=0, atol=1e-12)


def test_two_chunks_equal_one_prefill():
    """A sequence prefilled in two chunks (the second attending to the first
    through the cache) gives the rows of the one-shot causal prefill."""
    L, c = 150, 70
    q, K, V, kp, vp, table, _, _ = _pool_case(45, [L], [L], 4, 2, 8)
    cu_all = O.cu_seqlens_from_lengths([L])
    ro, rl = O.ragged_prefill(q, K[0], V[0], cu_all, 0.3)
    o1, l1 = O.chunk_prefill(q[:c], kp, vp, table, O.cu_seqlens_from_lengths([c]), np.array([c], np.int32), 0.3)
    o2, l2 = O.chunk_prefill(q[c:], kp, vp, table, O.cu_seqlens_from_lengths([L - c]), np.array([L], np.int32), 0.3)
    np.testing.assert_allclose(np.concatenate([o1, o2]), ro, rtol=0, atol=1e-12)
    np.testing.assert_allclose(np.concatenate([l1, l2]), rl, rtol=0, atol=1e-12)


def test_chunk_prefill_page_permutation_invariance_and_row_subset():
    kv_lens, q_lens = [190, 40], [60, 40]
    q, K, V, kp, vp, table, cu, kvl = _pool_case(46, kv_lens, q_lens, 4, 2, 8)
    out, lse = O.chunk_prefill(q, kp, vp, table, cu, kvl, 0.3)
    perm = np.random.default_rng(7).permutation(kp.shape[0])
    inv = np.argsort(perm)
    out2, lse2 = O.chunk_prefill(q, kp[perm], vp[perm], inv[table].astype(np.int32), cu, kvl, 0.3)
    np.testing.assert_array_equal(out, out2)
    np.testing.assert_array_equal(lse, lse2)
    rows = [0, 59, 60, 99]
    o3, l3 = O.chunk_prefill(q, kp, vp, table, cu, kvl, 0.3, rows=rows)
    np.testing.assert_array_equal(o3, out[rows])
    np.testing.assert_array_equal(l3, lse[rows])


def test_chunk_prefill_nan_outside_the_keys_never_leaks():
    """Rows past kv_len of the last block and unused blocks are NaN in the pool."""
    q, K, V, kp, vp, table, cu, kvl = _pool_case(47, [65, 3], [2, 3], 4, 4, 8)
    out, lse = O.chunk_prefill(q, kp, vp, table, cu, kvl, 0.3)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))


def test_chunk_first_query_of_a_new_sequence_returns_its_value_row():
    """kv_len == q_len: query 0 sees key 0 only, so out = V[0] exactly."""
    q, K, V, kp, vp, table, cu, kvl = _pool_case(48, [10], [10], 2, 1, 4)
    out, lse = O.chunk_prefill(q, kp, vp, table, cu, kvl, 0.5)
    np.testing.assert_array_equal(out[0, 0], V[0][0, 0])
    np.testing.assert_array_equal(out[0, 1], V[0][0, 0])
    np.testing.assert_allclose(lse[0, 0], 0.5 * q[0, 0] @ K[0][0, 0], rtol=0, atol=1e-14)


def test_empty_chunk_and_empty_cache():
    q, K, V, kp, vp, table, cu, kvl = _pool_case(49, [50, 1], [0, 1], 4, 2, 8)
    out, lse = O.chunk_prefill(q, kp, vp, table, cu, kvl, 0.3)
    assert out.shape == (1, 4, 8)
    np.testing.assert_array_equal(out[0, 0], V[1][0, 0])


def test_append_places_tokens_at_the_end_of_each_sequence():
    """After the append, gathering the kv_len logical rows reproduces the old
    prefix followed by the chunk, bit for bit, and nothing else changes."""
    rng = np.random.default_rng(50)
    B, Hk, D, NB = 3, 2, 8, 12
    kv_lens, q_lens = [70, 3, 128], [6, 3, 64]
    table = rng.permutation(NB)[: 3 * 2].reshape(3, 2).astype(np.int32)
    kp = rng.standard_normal((NB, Hk, 64, D))
    vp = rng.standard_normal((NB, Hk, 64, D))
    cu = O.cu_seqlens_from_lengths(q_lens)
    kn = rng.standard_normal((int(cu[-1]), Hk, D))
    vn = rng.standard_normal((int(cu[-1]), Hk, D))
    kp2, vp2 = O.append_kv(kn, vn, kp, vp, table, cu, np.array(kv_lens, np.int32))
    touched = np.zeros(kp.shape[:1] + (64,), bool)
    for b in range(B):
        first = kv_lens[b] - q_lens[b]
        for g in range(Hk):
            old = O.gather_kv_rows(kp, table, b, g, kv_lens[b])
            new = O.gather_kv_rows(kp2, table, b, g, kv_lens[b])
            np.testing.assert_array_equal(new[:first], old[:first])
            np.testing.assert_array_equal(new[first:], kn[cu[b]:cu[b + 1], g])
            np.testing.assert_array_equal(O.gather_kv_rows(vp2, table, b, g, kv_lens[b])[first:], vn[cu[b]:cu[b + 1], g])
        for p in range(first, kv_lens[b]):
            touched[table[b][p // 64], p % 64] = True
    rows = lambda x: x.transpose(0, 2, 1, 3)   # [NB, 64, Hk, D]: indexable by (block, row)
    np.testing.assert_array_equal(rows(kp2)[~touched], rows(kp)[~touched])
    np.testing.assert_array_equal(rows(vp2)[~touched], rows(vp)[~touched])


def test_append_then_chunk_prefill_equals_prefill_of_the_whole_sequence():
    """Fill the cache with the first 100 tokens, append the next 50 with the
    append rule, attend: the chunk's rows equal the one-shot prefill's."""
    rng = np.random.default_rng(51)
    L, c, Hq, Hk, D = 150, 100, 4, 2, 8
    table = np.array([[5, 1, 3]], np.int32)
    kp = np.full((6, Hk, 64, D), np.nan)
    vp = np.full((6, Hk, 64, D), np.nan)
    k = rng.standard_normal((L, Hk, D))
    v = rng.standard_normal((L, Hk, D))
    q = rng.standard_normal((L, Hq, D))
    kp, vp = O.append_kv(k[:c], v[:c], kp, vp, table, O.cu_seqlens_from_lengths([c]), np.array([c], np.int32))
    kp, vp = O.append_kv(k[c:], v[c:], kp, vp, table, O.cu_seqlens_from_lengths([L - c]), np.array([L], np.int32))
    o, l = O.chunk_prefill(q[c:], kp, vp, table, O.cu_seqlens_from_lengths([L - c]), np.array([L], np.int32), 0.3)
    ro, rl = O.ragged_prefill(q, k, v, O.cu_seqlens_from_lengths([L]), 0.3)
    np.testing.assert_allclose(o, ro[c:], rtol=0, atol=1e-12)
    np.testing.assert_allclose(l, rl[c:], rtol=0, atol=1e-12)


# ---------------------------------------------------------------- MLA: the rope key from the paged cache

def _mla_pool_case(seed, kv_lens, q_lens, Hq, Hk, Dn=8, Dr=4, Dv=6):
    """As _pool_case, plus a one-head rope cache [NB, 1, 64, Dr] on the same pages
    and queries of width Dn + Dr."""
    rng = np.random.default_rng(seed)
    B = len(kv_lens)
    nblk = max(1, max((L + 63) // 64 for L in kv_lens))
    NB = B * nblk + 2
    table = rng.permutation(NB)[: B * nblk].reshape(B, nblk).astype(np.int32)
    K = [rng.standard_normal((L, Hk, Dn)) for L in kv_lens]
    V = [rng.standard_normal((L, Hk, Dv)) for L in kv_lens]
    R = [rng.standard_normal((L, Dr)) for L in kv_lens]
    kp = np.full((NB, Hk, 64, Dn), np.nan)
    vp = np.full((NB, Hk, 64, Dv), np.nan)
    rp = np.full((NB, 1, 64, Dr), np.nan)
    for b, L in enumerate(kv_lens):
        for t in range(L):
            kp[table[b][t // 64], :, t % 64] = K[b][t]
            vp[table[b][t // 64], :, t % 64] = V[b][t]
            rp[table[b][t // 64], 0, t % 64] = R[b][t]
    cu = O.cu_seqlens_from_lengths(q_lens)
    q = rng.standard_normal((int(cu[-1]), Hq, Dn + Dr))
    return q, K, V, R, kp, vp, rp, table, cu, np.asarray(kv_lens, np.int32)


def test_mla_chunk_prefill_matches_bruteforce():
    kv_lens, q_lens = [70, 5, 130], [6, 5, 64]
    q, K, V, R, kp, vp, rp, table, cu, kvl = _mla_pool_case(71, kv_lens, q_lens, 4, 2)
    out, lse = O.chunk_prefill(q, kp, vp, table, cu, kvl, 0.3, kr_pool=rp)
    qs = [q[cu[b]:cu[b + 1]] for b in range(3)]
    bo, bl = BF.chunk_prefill(qs, K, V, [kv_lens[b] - q_lens[b] for b in range(3)], 0.3, k_rope=R)
    np.testing.assert_allclose(out, _cat(bo), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, _cat(bl), rtol=0, atol=1e-12)


def test_mla_chunk_with_empty_prefix_equals_mla_ragged_prefill():
    """No prefix: the MLA ragged prefill (rope rows given token-major) of the
    same logical tensors."""
    lens = [1, 64, 100]
    q, K, V, R, kp, vp, rp, table, cu, kvl = _mla_pool_case(72, lens, lens, 4, 4)
    out, lse = O.chunk_prefill(q, kp, vp, table, cu, kvl, 0.25, kr_pool=rp)
    ro, rl = O.ragged_prefill(q, np.concatenate(K), np.concatenate(V), cu, 0.25,
                              k_rope=np.concatenate(R)[:, None, :])
    np.testing.assert_allclose(out, ro, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, rl, rtol=0, atol=1e-12)


def test_mla_chunk_zero_rope_query_reduces_to_plain_chunk():
    """Zeroing the rope part of the queries removes the rope term exactly."""
    q, K, V, R, kp, vp, rp, table, cu, kvl = _mla_pool_case(73, [150, 20], [40, 20], 4, 2)
    q[:, :, 8:] = 0.0
    out, lse = O.chunk_prefill(q, kp, vp, table, cu, kvl, 0.3, kr_pool=rp)
    po, pl = O.chunk_prefill(q[:, :, :8], kp, vp, table, cu, kvl, 0.3)
    np.testing.assert_allclose(out, po, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, pl, rtol=0, atol=1e-14)


def test_mla_append_writes_the_rope_rows_on_the_same_pages():
    q, K, V, R, kp, vp, rp, table, cu, kvl = _mla_pool_case(74, [130, 64], [64, 1], 4, 2)
    T = int(cu[-1])
    rng = np.random.default_rng(75)
    kn, vn, rn = rng.standard_normal((T, 2, 8)), rng.standard_normal((T, 2, 6)), rng.standard_normal((T, 1, 4))
    kp2, vp2, rp2 = O.append_kv(kn, vn, kp, vp, table, cu, kvl, kr_new=rn, kr_pool=rp)
    for b, (L, n) in enumerate(((130, 64), (64, 1))):
        got = O.gather_kv_rows(rp2, table, b, 0, L)
        np.testing.assert_array_equal(got[: L - n], R[b][: L - n])
        np.testing.assert_array_equal(got[L - n:], rn[cu[b]:cu[b + 1], 0])


# ---------------------------------------------------------------- CSR page input

def test_csr_block_table_round_trip_and_decode_equivalence():
    """A padded table written out as (kv_indices, kv_page_indptr) -- each
    sequence's used pages in order, indptr the prefix of the page counts
    ceil(L / 64) -- and read back gives the used entries of the original
    table and -1 padding, so decode through it is unchanged."""
    rng = np.random.default_rng(80)
    B, Hq, Hk, D = 4, 4, 2, 8
    lens = [130, 0, 64, 5]
    nblk, NB = 3, 12
    table = rng.permutation(NB)[: B * nblk].reshape(B, nblk).astype(np.int32)
    counts = [(L + 63) // 64 for L in lens]
    kv_indices = np.concatenate([table[b, :counts[b]] for b in range(B)]).astype(np.int32)
    indptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    back = O.block_table_from_csr(kv_indices, indptr, nblk)
    for b in range(B):
        np.testing.assert_array_equal(back[b, :counts[b]], table[b, :counts[b]])
        assert np.all(back[b, counts[b]:] == -1)
    q = rng.standard_normal((B, Hq, D))
    kp = rng.standard_normal((NB, Hk, 64, D))
    vp = rng.standard_normal((NB, Hk, 64, D))
    sl = np.array(lens, np.int32)
    o1, l1 = O.paged_decode(q, kp, vp, table, sl, 0.3)
    o2, l2 = O.paged_decode(q, kp, vp, back, sl, 0.3)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_csr_block_table_follows_the_flat_index_order():
    """Hand example: three sequences with 2, 0 and 3 pages."""
    t = O.block_table_from_csr(np.array([7, 3, 9, 1, 4], np.int32), np.array([0, 2, 2, 5], np.int32), 4)
    np.testing.assert_array_equal(t, [[7, 3, -1, -1], [-1, -1, -1, -1], [9, 1, 4, -1]])
