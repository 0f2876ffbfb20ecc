"""Pins for the CPU oracle: brute force, library routines, closed forms,
invariants and the pages' own printed mappings.  CPU only."""
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import attention as O
from oracle import bruteforce as BF
from workloads import gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# helpers (test-local; written from the pages' mapping, independent of the oracle)
# --------------------------------------------------------------------------

def _scatter(logical, seq_lens, block_table, NB):
    """Place logical rows logical[b] ([Hk, L_b, D]) into a NaN pool [NB, Hk, 64, D]:
    token t goes to block block_table[b][t // 64], row t - 64 * (t // 64)."""
    Hk, D = logical[0].shape[0], logical[0].shape[2]
    pool = np.full((NB, Hk, 64, D), np.nan)
    for b, L in enumerate(seq_lens):
        for t in range(L):
            col = t // 64
            pool[int(block_table[b][col]), :, t - 64 * col, :] = logical[b][:, t, :]
    return pool


def _tiny_decode(seed, B, Hq, Hk, D, seq_lens, extra_blocks=3):
    rng = np.random.default_rng(seed)
    nblk = max(1, max((L + 63) // 64 for L in seq_lens))
    NB = B * nblk + extra_blocks
    table = rng.permutation(NB)[: B * nblk].reshape(B, nblk).astype(np.int32)
    q = rng.standard_normal((B, Hq, D))
    K = [rng.standard_normal((Hk, L, D)) for L in seq_lens]
    V = [rng.standard_normal((Hk, L, D)) for L in seq_lens]
    kp = _scatter(K, seq_lens, table, NB)
    vp = _scatter(V, seq_lens, table, NB)
    return q, K, V, kp, vp, table, np.asarray(seq_lens, np.int32)


def _sdpa_decode(q, K, V, seq_lens, scale):
    """torch fp64 scaled_dot_product_attention on unpaged, head-expanded keys."""
    B, Hq, D = q.shape
    outs, lses = [], []
    for b in range(B):
        Hk = K[b].shape[0]
        r = Hq // Hk
        Kb = torch.from_numpy(K[b]).repeat_interleave(r, dim=0)   # [Hq, L, D]
        Vb = torch.from_numpy(V[b]).repeat_interleave(r, dim=0)
        qb = torch.from_numpy(q[b])[:, None, :]                    # [Hq, 1, D]
        o = F.scaled_dot_product_attention(qb, Kb, Vb, scale=scale)[:, 0]
        s = scale * torch.matmul(qb, Kb.transpose(-1, -2).contiguous())[:, 0]
        outs.append(o.numpy())
        lses.append(torch.logsumexp(s, dim=-1).numpy())
    return np.stack(outs), np.stack(lses)


def _tiny_prefill(seed, lens, Hq, Hk, Dn, Dr, Dv):
    rng = np.random.default_rng(seed)
    T = sum(lens)
    q = rng.standard_normal((T, Hq, Dn + Dr))
    k = rng.standard_normal((T, Hk, Dn))
    v = rng.standard_normal((T, Hk, Dv))
    kr = rng.standard_normal((T, 1, Dr)) if Dr else None
    return q, k, v, kr, O.cu_seqlens_from_lengths(lens)


def _split(x, cu):
    return [x[cu[b]:cu[b + 1]] for b in range(len(cu) - 1)]


# --------------------------------------------------------------------------
# storage formats
# --------------------------------------------------------------------------

def test_e4m3fn_table_matches_torch_all_codes():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.e4m3fn_table(), ref)   # NaN positions must agree too


def test_e4m3fn_closed_form_points():
    # OCP E4M3FN: bias 7, 3 mantissa bits, no inf, S.1111.111 is NaN.
    t = O.e4m3fn_table()
    assert t[0x38] == 1.0 and t[0xB8] == -1.0
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0          # largest finite
    assert t[0x08] == 2.0 ** -6                             # smallest normal
    assert t[0x01] == 2.0 ** -9                             # smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9                         # largest subnormal
    assert math.isnan(t[0x7F]) and math.isnan(t[0xFF])
    assert t[0x00] == 0.0 and math.copysign(1.0, t[0x80]) == -1.0
    assert np.isnan(t).sum() == 2


def test_bf16_widen_matches_torch():
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 1 << 16, 20000, dtype=np.uint32).astype(np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]               # finite values only
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.bf16_to_f64(bits), ref)


# --------------------------------------------------------------------------
# paged decode
# --------------------------------------------------------------------------

@pytest.mark.parametrize("Hq,Hk", [(6, 2), (8, 4), (4, 4)])
def test_decode_matches_bruteforce_on_unpaged_tensors(Hq, Hk):
    seq_lens = [1, 70, 130]
    q, K, V, kp, vp, table, sl = _tiny_decode(11, 3, Hq, Hk, 8, seq_lens)
    out, lse = O.paged_decode(q, kp, vp, table, sl, 0.37)
    bo, bl = BF.decode(q, K, V, sl, 0.37, Hk)
    np.testing.assert_allclose(out, np.array(bo), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, np.array(bl), rtol=0, atol=1e-12)


def test_decode_matches_torch_sdpa():
    seq_lens = [5, 64, 65, 200, 129]
    q, K, V, kp, vp, table, sl = _tiny_decode(12, 5, 16, 4, 32, seq_lens)
    out, lse = O.paged_decode(q, kp, vp, table, sl, 1 / math.sqrt(32))
    so, sle = _sdpa_decode(q, K, V, sl, 1 / math.sqrt(32))
    np.testing.assert_allclose(out, so, rtol=0, atol=1e-10)
    np.testing.assert_allclose(lse, sle, rtol=0, atol=1e-10)


def test_decode_block_shuffle_leaves_output_unchanged():
    c = gen.make_decode_case(name="t", seed=5, B=4, Hq=8, Hk=2, D=16, q_dtype="bf16",
                             kv_dtype="bf16", seq_lens=[3, 64, 100, 191])
    args = dict(q_dtype="bf16", kv_dtype="bf16")
    out, lse = O.paged_decode(c.q, c.k_pool, c.v_pool, c.block_table, c.seq_lens, c.scale, **args)
    perm = np.random.default_rng(9).permutation(c.NB)
    kp2 = np.empty_like(c.k_pool)
    vp2 = np.empty_like(c.v_pool)
    kp2[perm] = c.k_pool
    vp2[perm] = c.v_pool
    t2 = np.where(c.block_table >= 0, perm[np.maximum(c.block_table, 0)], -1).astype(np.int32)
    out2, lse2 = O.paged_decode(c.q, kp2, vp2, t2, c.seq_lens, c.scale, **args)
    np.testing.assert_array_equal(out, out2)
    np.testing.assert_array_equal(lse, lse2)


def test_decode_seq_len_one_returns_that_v_row():
    q, K, V, kp, vp, table, sl = _tiny_decode(13, 2, 4, 2, 16, [1, 1])
    out, lse = O.paged_decode(q, kp, vp, table, sl, 0.25)
    for b in range(2):
        for h in range(4):
            np.testing.assert_array_equal(out[b, h], V[b][h // 2][0])


def test_decode_head_mapping_matches_page_diagram():
    pairs = np.loadtxt(os.path.join(GOLDEN, "gqa_head_map_hq8_hk4.txt"), dtype=int)
    seq_lens = [70, 9]
    q, K, V, kp, vp, table, sl = _tiny_decode(14, 2, 8, 4, 8, seq_lens)
    V = [np.broadcast_to((np.arange(4) + 1.0)[:, None, None], v.shape).copy() for v in V]
    vp = _scatter(V, seq_lens, table, kp.shape[0])
    out, _ = O.paged_decode(q, kp, vp, table, sl, 0.3)
    for qh, kvh in pairs:
        # a weighted mean of a constant row is that constant up to summation rounding
        np.testing.assert_allclose(out[:, qh, :], kvh + 1.0, rtol=0, atol=1e-12, err_msg=str((qh, kvh)))


def test_decode_ignores_nan_tails_and_unused_blocks():
    c = gen.decode_tiny_fp32()
    out, lse = O.paged_decode(c.q, c.k_pool, c.v_pool, c.block_table, c.seq_lens, c.scale,
                              q_dtype="f32", kv_dtype="f32")
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    # replacing every poisoned slot by finite junk must not change anything
    kp = np.where(np.isnan(c.k_pool), np.float32(1e3), c.k_pool)
    vp = np.where(np.isnan(c.v_pool), np.float32(-7.0), c.v_pool)
    out2, lse2 = O.paged_decode(c.q, kp, vp, c.block_table, c.seq_lens, c.scale,
                                q_dtype="f32", kv_dtype="f32")
    np.testing.assert_array_equal(out, out2)
    np.testing.assert_array_equal(lse, lse2)


def test_decode_zero_query_gives_mean_of_values():
    seq_lens = [7, 130]
    q, K, V, kp, vp, table, sl = _tiny_decode(15, 2, 4, 2, 8, seq_lens)
    q[:] = 0.0
    out, lse = O.paged_decode(q, kp, vp, table, sl, 0.5)
    for b, L in enumerate(seq_lens):
        for h in range(4):
            np.testing.assert_allclose(out[b, h], V[b][h // 2].mean(axis=0), rtol=0, atol=1e-14)
            assert abs(lse[b, h] - math.log(L)) < 1e-14


def test_decode_empty_sequence():
    q, K, V, kp, vp, table, sl = _tiny_decode(16, 2, 4, 2, 8, [0, 5])
    out, lse = O.paged_decode(q, kp, vp, table, sl, 0.5)
    assert np.all(out[0] == 0.0) and np.all(np.isneginf(lse[0]))
    assert np.isfinite(out[1]).all()


def test_decode_fp8_matches_sdpa_on_torch_dequantised_cache():
    c = gen.make_decode_case(name="t", seed=21, B=3, Hq=8, Hk=2, D=32, q_dtype="bf16",
                             kv_dtype="e4m3fn", seq_lens=[10, 64, 150])
    out, lse = O.paged_decode(c.q, c.k_pool, c.v_pool, c.block_table, c.seq_lens, c.scale,
                              q_dtype="bf16", kv_dtype="e4m3fn", k_scale=c.k_scale, v_scale=c.v_scale)
    # independent decoding: torch's float8_e4m3fn -> float64 and an explicit per-token gather loop
    q = torch.from_numpy(c.q.view(np.int16)).view(torch.bfloat16).double().numpy()
    kf = torch.from_numpy(c.k_pool).view(torch.float8_e4m3fn).double().numpy() * c.k_scale
    vf = torch.from_numpy(c.v_pool).view(torch.float8_e4m3fn).double().numpy() * c.v_scale
    K, V = [], []
    for b, L in enumerate(c.seq_lens):
        K.append(np.stack([kf[c.block_table[b, t // 64], :, t % 64] for t in range(L)], axis=1))
        V.append(np.stack([vf[c.block_table[b, t // 64], :, t % 64] for t in range(L)], axis=1))
    so, sle = _sdpa_decode(q, K, V, c.seq_lens, c.scale)
    np.testing.assert_allclose(out, so, rtol=0, atol=1e-10)
    np.testing.assert_allclose(lse, sle, rtol=0, atol=1e-10)


def test_gather_follows_page_token_block_mapping():
    rows = np.loadtxt(os.path.join(GOLDEN, "prefill_token_blocks.txt"), dtype=int)
    NB, D = 9, 4
    pool = np.zeros((NB, 1, 64, D))
    for blk in range(NB):
        for r in range(64):
            pool[blk, 0, r, :] = 1000 * blk + r
    table = np.array([[7, 3, 5]], np.int32)
    got = O.gather_kv_rows(pool, table, 0, 0, 192)
    for first, last, col in rows:
        for t in range(first, last + 1):
            assert got[t, 0] == 1000 * table[0, col] + (t - first), t


# --------------------------------------------------------------------------
# ragged prefill
# --------------------------------------------------------------------------

def test_prefill_matches_bruteforce_with_rope():
    lens = [3, 70, 130]
    q, k, v, kr, cu = _tiny_prefill(31, lens, 4, 2, 8, 4, 6)
    out, lse = O.ragged_prefill(q, k, v, cu, 0.3, k_rope=kr)
    bo, bl = BF.prefill(_split(q, cu), _split(k, cu), _split(v, cu), lens, 0.3,
                        k_rope=[x[:, 0, :] for x in _split(kr, cu)])
    np.testing.assert_allclose(out, np.concatenate([np.array(x) for x in bo]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, np.concatenate([np.array(x) for x in bl]), rtol=0, atol=1e-12)


def test_prefill_matches_bruteforce_with_block_mask():
    lens = [150, 40]
    q, k, v, _, cu = _tiny_prefill(32, lens, 4, 1, 6, 0, 5)
    mask = np.array([[[1, 0, 0], [0, 1, 0], [1, 1, 0]],
                     [[0, 0, 0], [1, 1, 0], [1, 1, 1]]], np.uint8)   # seq 1 block 0 fully off
    out, lse = O.ragged_prefill(q, k, v, cu, 0.4, block_mask=mask)
    bo, bl = BF.prefill(_split(q, cu), _split(k, cu), _split(v, cu), lens, 0.4, block_mask=mask)
    np.testing.assert_allclose(out, np.concatenate([np.array(x) for x in bo]), rtol=0, atol=1e-12)
    np.testing.assert_array_equal(np.isneginf(lse), np.isneginf(np.concatenate([np.array(x) for x in bl])))
    fin = np.isfinite(lse)
    np.testing.assert_allclose(lse[fin], np.concatenate([np.array(x) for x in bl])[fin], rtol=0, atol=1e-12)
    # the fully-masked rows (sequence 1, first block) are zero with lse -inf
    assert np.all(out[150:190] == 0.0) and np.all(np.isneginf(lse[150:190]))


def _sdpa_prefill(q, k, v, kr, cu, scale, elem_masks=None):
    outs = []
    Hq, Hk = q.shape[1], k.shape[1]
    r = Hq // Hk
    for b in range(len(cu) - 1):
        sl = slice(cu[b], cu[b + 1])
        kb = k[sl]
        if kr is not None:
            kb = np.concatenate([kb, np.broadcast_to(kr[sl], (kb.shape[0], Hk, kr.shape[2]))], axis=2)
        K = torch.from_numpy(np.ascontiguousarray(kb.transpose(1, 0, 2))).repeat_interleave(r, 0)
        V = torch.from_numpy(np.ascontiguousarray(v[sl].transpose(1, 0, 2))).repeat_interleave(r, 0)
        Q = torch.from_numpy(np.ascontiguousarray(q[sl].transpose(1, 0, 2)))
        if elem_masks is None:
            o = F.scaled_dot_product_attention(Q, K, V, is_causal=True, scale=scale)
        else:
            o = F.scaled_dot_product_attention(Q, K, V, attn_mask=torch.from_numpy(elem_masks[b]), scale=scale)
        outs.append(o.numpy().transpose(1, 0, 2))
    return np.concatenate(outs)


def test_prefill_mla_matches_sdpa_with_concatenated_rope_key():
    lens = [64, 100, 1, 200]
    q, k, v, kr, cu = _tiny_prefill(33, lens, 4, 4, 16, 8, 16)
    out, _ = O.ragged_prefill(q, k, v, cu, 1 / math.sqrt(24), k_rope=kr)
    np.testing.assert_allclose(out, _sdpa_prefill(q, k, v, kr, cu, 1 / math.sqrt(24)), rtol=0, atol=1e-10)


def test_prefill_gqa_matches_sdpa():
    lens = [130, 77]
    q, k, v, _, cu = _tiny_prefill(34, lens, 8, 2, 16, 0, 16)
    out, _ = O.ragged_prefill(q, k, v, cu, 0.25)
    np.testing.assert_allclose(out, _sdpa_prefill(q, k, v, None, cu, 0.25), rtol=0, atol=1e-10)


def test_prefill_block_mask_matches_sdpa_element_mask():
    lens = [200, 129]
    q, k, v, _, cu = _tiny_prefill(35, lens, 4, 2, 8, 0, 8)
    rng = np.random.default_rng(1)
    mask = np.tril((rng.random((2, 4, 4)) < 0.5)).astype(np.uint8)
    mask[:, np.arange(4), np.arange(4)] = 1        # keep every row non-empty for SDPA
    elem = []
    for b, L in enumerate(lens):
        em = np.kron(mask[b], np.ones((64, 64), np.uint8))[:L, :L].astype(bool)
        elem.append(em & np.tril(np.ones((L, L), bool)))
    out, _ = O.ragged_prefill(q, k, v, cu, 0.3, block_mask=mask)
    np.testing.assert_allclose(out, _sdpa_prefill(q, k, v, None, cu, 0.3, elem_masks=elem), rtol=0, atol=1e-10)


def test_prefill_all_on_block_mask_equals_dense():
    lens = [150, 64]
    q, k, v, _, cu = _tiny_prefill(36, lens, 4, 2, 8, 0, 8)
    out, lse = O.ragged_prefill(q, k, v, cu, 0.3)
    ones = np.ones((2, 3, 3), np.uint8)
    out2, lse2 = O.ragged_prefill(q, k, v, cu, 0.3, block_mask=ones)
    np.testing.assert_array_equal(out, out2)
    np.testing.assert_array_equal(lse, lse2)


def test_prefill_diagonal_only_mask_equals_independent_64_token_sequences():
    q, k, v, _, cu = _tiny_prefill(37, [192], 4, 2, 8, 0, 8)
    eye = np.eye(3, dtype=np.uint8)[None]
    out, _ = O.ragged_prefill(q, k, v, cu, 0.3, block_mask=eye)
    out2, _ = O.ragged_prefill(q, k, v, np.array([0, 64, 128, 192], np.int32), 0.3)
    # same terms; only the number of zero-weight terms in each sum differs
    np.testing.assert_allclose(out, out2, rtol=0, atol=1e-14)


def test_prefill_packed_equals_each_sequence_alone():
    lens = [70, 5, 131]
    q, k, v, kr, cu = _tiny_prefill(38, lens, 4, 2, 8, 4, 8)
    out, lse = O.ragged_prefill(q, k, v, cu, 0.3, k_rope=kr)
    for b, L in enumerate(lens):
        sl = slice(cu[b], cu[b + 1])
        o1, l1 = O.ragged_prefill(q[sl], k[sl], v[sl], np.array([0, L]), 0.3, k_rope=kr[sl])
        np.testing.assert_array_equal(out[sl], o1)
        np.testing.assert_array_equal(lse[sl], l1)


def test_prefill_row_subset_equals_full():
    lens = [100, 60]
    q, k, v, kr, cu = _tiny_prefill(39, lens, 4, 2, 8, 4, 8)
    out, lse = O.ragged_prefill(q, k, v, cu, 0.3, k_rope=kr)
    rows = np.array([0, 17, 99, 100, 159])
    o2, l2 = O.ragged_prefill(q, k, v, cu, 0.3, k_rope=kr, rows=rows)
    np.testing.assert_array_equal(out[rows], o2)
    np.testing.assert_array_equal(lse[rows], l2)


def test_prefill_zero_rope_query_reduces_to_nope_attention():
    lens = [90]
    q, k, v, kr, cu = _tiny_prefill(40, lens, 4, 4, 8, 4, 8)
    q[:, :, 8:] = 0.0
    out, _ = O.ragged_prefill(q, k, v, cu, 0.3, k_rope=kr)
    out2, _ = O.ragged_prefill(np.ascontiguousarray(q[:, :, :8]), k, v, cu, 0.3)
    np.testing.assert_allclose(out, out2, rtol=0, atol=1e-14)


def test_prefill_first_row_returns_its_own_value_row():
    lens = [10, 3]
    q, k, v, kr, cu = _tiny_prefill(41, lens, 4, 2, 8, 4, 8)
    out, _ = O.ragged_prefill(q, k, v, cu, 0.3, k_rope=kr)
    for b in range(2):
        for h in range(4):
            np.testing.assert_array_equal(out[cu[b], h], v[cu[b], h // 2])


def test_generated_configs_flops_and_bytes():
    # the MLA prefill numerator has a closed form: 2*Hq*(192+128)*sum L(L+1)/2
    p = gen.prefill_mla_bf16()
    lens = [512, 1024, 2048, 3000]
    assert p.flops() == 2 * 16 * 320 * sum(L * (L + 1) // 2 for L in lens)
    assert list(p.cu_seqlens) == [0, 512, 1536, 3584, 6584]
