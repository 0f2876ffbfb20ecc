"""Pins for the oracle's fp8 prefill (q_nope and K as e4m3fn codes with one
scale per tensor or one per row of a head, rope parts and V in bf16).  CPU only.

Each pin decodes the codes with torch's own float8_e4m3fn and bfloat16 types
(not the oracle's tables) and checks the oracle against plain-Python brute
force, torch's scaled_dot_product_attention, an exact invariance of the scales,
or a case where the answer is known without the nope part."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import attention as O
from oracle import bruteforce as BF
from workloads import gen


def _codes(rng, shape):
    """Random e4m3fn codes, NaN codes (0x7F, 0xFF) excluded."""
    c = rng.integers(0, 256, size=shape, dtype=np.int64).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x7E
    return c


def _bf16(rng, shape):
    return gen.to_bf16_bits(rng.standard_normal(shape).astype(np.float32))


def _t8(c):
    return torch.from_numpy(c).view(torch.float8_e4m3fn).double().numpy()


def _tb(b):
    return torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).double().numpy()


def _case(seed, lens, Hq, Hk, Dn, Dr, Dv):
    rng = np.random.default_rng(seed)
    T = sum(lens)
    qn = _codes(rng, (T, Hq, Dn))
    k = _codes(rng, (T, Hk, Dn))
    qr = _bf16(rng, (T, Hq, Dr)) if Dr else None
    kr = _bf16(rng, (T, 1, Dr)) if Dr else None
    v = _bf16(rng, (T, Hk, Dv))
    return qn, qr, k, v, kr, O.cu_seqlens_from_lengths(lens)


def _split(x, cu):
    return [x[cu[b]:cu[b + 1]] for b in range(len(cu) - 1)]


def test_fp8_prefill_matches_bruteforce_on_torch_decoded_codes():
    lens = [3, 70, 130]
    qs, ks, sc = 0.0123, 0.0371, 0.29
    qn, qr, k, v, kr, cu = _case(71, lens, 4, 2, 8, 4, 6)
    out, lse = O.ragged_prefill_fp8(qn, qr, k, v, kr, cu, sc, qs, ks)
    q = np.concatenate([_t8(qn) * qs, _tb(qr)], axis=2)
    bo, bl = BF.prefill(_split(q, cu), _split(_t8(k) * ks, cu), _split(_tb(v), cu), lens, sc,
                        k_rope=[x[:, 0, :] for x in _split(_tb(kr), cu)])
    np.testing.assert_allclose(out, np.concatenate([np.array(x) for x in bo]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, np.concatenate([np.array(x) for x in bl]), rtol=0, atol=1e-12)


def test_fp8_prefill_matches_sdpa_with_concatenated_rope_key():
    lens = [64, 100, 1, 150]
    qs, ks, sc = 0.02, 0.05, 1 / math.sqrt(24)
    qn, qr, k, v, kr, cu = _case(72, lens, 4, 4, 16, 8, 16)
    out, _ = O.ragged_prefill_fp8(qn, qr, k, v, kr, cu, sc, qs, ks)
    ref = []
    for b in range(len(lens)):
        s = slice(cu[b], cu[b + 1])
        Q = np.concatenate([_t8(qn[s]) * qs, _tb(qr[s])], axis=2).transpose(1, 0, 2)
        K = np.concatenate([_t8(k[s]) * ks, np.broadcast_to(_tb(kr[s]), (lens[b], 4, 8))], axis=2).transpose(1, 0, 2)
        V = _tb(v[s]).transpose(1, 0, 2)
        o = F.scaled_dot_product_attention(torch.from_numpy(np.ascontiguousarray(Q)),
                                           torch.from_numpy(np.ascontiguousarray(K)),
                                           torch.from_numpy(np.ascontiguousarray(V)), is_causal=True, scale=sc)
        ref.append(o.numpy().transpose(1, 0, 2))
    np.testing.assert_allclose(out, np.concatenate(ref), rtol=0, atol=1e-10)


def test_fp8_prefill_gqa_without_rope_matches_sdpa():
    lens = [130, 77]
    qs, ks, sc = 0.011, 0.013, 0.25
    qn, _, k, v, _, cu = _case(73, lens, 8, 2, 16, 0, 16)
    out, _ = O.ragged_prefill_fp8(qn, None, k, v, None, cu, sc, qs, ks)
    ref = []
    for b in range(len(lens)):
        s = slice(cu[b], cu[b + 1])
        Q = torch.from_numpy(np.ascontiguousarray((_t8(qn[s]) * qs).transpose(1, 0, 2)))
        K = torch.from_numpy(np.ascontiguousarray((_t8(k[s]) * ks).transpose(1, 0, 2))).repeat_interleave(4, 0)
        V = torch.from_numpy(np.ascontiguousarray(_tb(v[s]).transpose(1, 0, 2))).repeat_interleave(4, 0)
        ref.append(F.scaled_dot_product_attention(Q, K, V, is_causal=True, scale=sc).numpy().transpose(1, 0, 2))
    np.testing.assert_allclose(out, np.concatenate(ref), rtol=0, atol=1e-10)


def test_fp8_prefill_only_the_scale_product_matters():
    """(q_scale * 8, k_scale / 8) gives exactly the result of (q_scale, k_scale):
    powers of two move between the factors without rounding."""
    lens = [90, 40]
    qn, qr, k, v, kr, cu = _case(74, lens, 4, 2, 16, 8, 8)
    a = O.ragged_prefill_fp8(qn, qr, k, v, kr, cu, 0.2, 0.03, 0.07)
    b = O.ragged_prefill_fp8(qn, qr, k, v, kr, cu, 0.2, 0.03 * 8, 0.07 / 8)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_fp8_prefill_scales_leave_the_rope_part_alone():
    """With every q_nope code zero the nope term vanishes, so the result is
    rope-only attention and does not depend on q_scale or k_scale; a scale
    applied to the whole score would change it."""
    lens = [70, 33]
    qn, qr, k, v, kr, cu = _case(75, lens, 4, 4, 16, 8, 8)
    qn[:] = 0
    a = O.ragged_prefill_fp8(qn, qr, k, v, kr, cu, 0.3, 0.5, 4.0)
    b = O.ragged_prefill_fp8(qn, qr, k, v, kr, cu, 0.3, 0.01, 0.02)
    np.testing.assert_array_equal(a[0], b[0])
    bo, _ = BF.prefill(_split(_tb(qr), cu), _split(np.zeros((sum(lens), 4, 0)), cu), _split(_tb(v), cu), lens, 0.3,
                       k_rope=[x[:, 0, :] for x in _split(_tb(kr), cu)])
    np.testing.assert_allclose(a[0], np.concatenate([np.array(x) for x in bo]), rtol=0, atol=1e-12)


def test_fp8_prefill_first_row_returns_its_own_value_row():
    lens = [5, 9]
    qn, qr, k, v, kr, cu = _case(76, lens, 2, 1, 16, 8, 8)
    out, _ = O.ragged_prefill_fp8(qn, qr, k, v, kr, cu, 0.3, 0.1, 0.1)
    for b in range(2):
        np.testing.assert_array_equal(out[cu[b]], np.repeat(_tb(v[cu[b]]), 2, axis=0))


def test_fp8_prefill_rope_args_go_together():
    qn, qr, k, v, kr, cu = _case(77, [4], 2, 2, 16, 8, 8)
    with pytest.raises(ValueError):
        O.ragged_prefill_fp8(qn, qr, k, v, None, cu, 0.3, 1.0, 1.0)


def test_fp8_prefill_generator_recipe():
    """The fp8 case is the bf16 case of the same seed, quantised: q_rope, K_rope
    and V are the same bits, the scales are amax/448 of the bf16 values, and
    the codes decode to within half an fp8 step of them."""
    lens = [70, 200]
    c8 = gen.make_prefill_fp8_case(name="t", seed=5, seq_lens=lens, Hq=4, Hk=2, D_rope=64)
    cb = gen.make_prefill_case(name="t", seed=5, seq_lens=lens, Hq=4, Hk=2, D_qk=192, D_rope=64, D_v=128)
    assert c8.dtype == "e4m3fn" and c8.q.dtype == np.uint8 and c8.k.dtype == np.uint8
    assert c8.q.shape == (270, 4, 128) and c8.q_rope.shape == (270, 4, 64) and c8.k.shape == (270, 2, 128)
    np.testing.assert_array_equal(c8.q_rope, cb.q[:, :, 128:])
    np.testing.assert_array_equal(c8.v, cb.v)
    np.testing.assert_array_equal(c8.k_rope, cb.k_rope)
    for codes, bits, sc in ((c8.q, cb.q[:, :, :128], c8.q_scale), (c8.k, cb.k, c8.k_scale)):
        x = _tb(np.ascontiguousarray(bits))
        assert sc == pytest.approx(np.abs(x).max() / 448, rel=1e-6)
        assert not np.any((codes & 0x7F) == 0x7F)
        err = np.abs(_t8(codes) * sc - x)
        assert np.all(err <= np.abs(x) * 2.0 ** -4 + sc * 2.0 ** -10)


# ---------------------------------------------------------------- blockwise scales (one per row of a head)

def test_fp8_blockwise_matches_bruteforce_on_torch_decoded_codes():
    lens = [3, 70, 130]
    T = sum(lens)
    rng = np.random.default_rng(78)
    qs = rng.uniform(0.005, 0.05, size=(T, 4)).astype(np.float32)
    ks = rng.uniform(0.005, 0.05, size=(T, 2)).astype(np.float32)
    qn, qr, k, v, kr, cu = _case(79, lens, 4, 2, 8, 4, 6)
    out, lse = O.ragged_prefill_fp8(qn, qr, k, v, kr, cu, 0.29, qs, ks)
    q = np.concatenate([_t8(qn) * qs.astype(np.float64)[:, :, None], _tb(qr)], axis=2)
    kv = _t8(k) * ks.astype(np.float64)[:, :, None]
    bo, bl = BF.prefill(_split(q, cu), _split(kv, cu), _split(_tb(v), cu), lens, 0.29,
                        k_rope=[x[:, 0, :] for x in _split(_tb(kr), cu)])
    np.testing.assert_allclose(out, np.concatenate([np.array(x) for x in bo]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, np.concatenate([np.array(x) for x in bl]), rtol=0, atol=1e-12)


def test_fp8_blockwise_with_equal_scales_is_the_per_tensor_result():
    lens = [90, 40]
    qn, qr, k, v, kr, cu = _case(80, lens, 4, 2, 16, 8, 8)
    a = O.ragged_prefill_fp8(qn, qr, k, v, kr, cu, 0.2, 0.03, 0.07)
    b = O.ragged_prefill_fp8(qn, qr, k, v, kr, cu, 0.2, np.full((130, 4), 0.03), np.full((130, 2), 0.07))
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_fp8_blockwise_key_scale_zero_removes_the_nope_term_of_that_key():
    """k_scale[j] = 0 leaves key j only its rope score: the result equals the
    oracle with that key's codes zeroed (a different input, same definition)."""
    lens = [40]
    qn, qr, k, v, kr, cu = _case(81, lens, 2, 1, 16, 8, 8)
    ks = np.full((40, 1), 0.04)
    ks[[3, 17, 39]] = 0.0
    a = O.ragged_prefill_fp8(qn, qr, k, v, kr, cu, 0.3, 0.02, ks)
    k0 = k.copy()
    k0[[3, 17, 39]] = 0
    b = O.ragged_prefill_fp8(qn, qr, k0, v, kr, cu, 0.3, 0.02, 0.04)
    np.testing.assert_allclose(a[0], b[0], rtol=0, atol=1e-14)


def test_fp8_blockwise_generator_recipe():
    lens = [70, 200]
    c8 = gen.make_prefill_fp8_case(name="t", seed=6, seq_lens=lens, Hq=4, Hk=2, D_rope=64, blockwise=True)
    cb = gen.make_prefill_case(name="t", seed=6, seq_lens=lens, Hq=4, Hk=2, D_qk=192, D_rope=64, D_v=128)
    assert c8.q_scale.shape == (270, 4) and c8.k_scale.shape == (270, 2)
    assert c8.q_scale.dtype == np.float32 and c8.k_scale.dtype == np.float32
    for codes, bits, sc in ((c8.q, cb.q[:, :, :128], c8.q_scale), (c8.k, cb.k, c8.k_scale)):
        x = _tb(np.ascontiguousarray(bits))
        np.testing.assert_allclose(sc, np.abs(x).max(axis=2) / 448, rtol=1e-6)
        err = np.abs(_t8(codes) * sc.astype(np.float64)[:, :, None] - x)
        assert np.all(err <= np.abs(x) * 2.0 ** -4 + sc[:, :, None] * 2.0 ** -10)
        # every row uses its full range: its largest code is +-448
        assert np.all(np.abs(_t8(codes)).max(axis=2) == 448)
