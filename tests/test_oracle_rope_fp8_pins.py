"""Pins for the oracle's MLA prefill with a quantised shared rope key (the
rope rows as e4m3fn codes with one scale per row; q, k and v bf16).  CPU only.

Each pin decodes the codes with torch's own float8_e4m3fn and bfloat16 types
(not the oracle's tables) and checks the oracle against plain-Python brute
force, torch's scaled_dot_product_attention, a case where the rope term
vanishes and the scales must not matter, power-of-two scales that make the
rope key an exact bf16 tensor, and zero scales that must act like zero codes
row by row."""
import math

import numpy as np
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
    q = _bf16(rng, (T, Hq, Dn + Dr))
    k = _bf16(rng, (T, Hk, Dn))
    v = _bf16(rng, (T, Hk, Dv))
    kr = _codes(rng, (T, 1, Dr))
    ks = (rng.uniform(0.002, 0.05, size=T)).astype(np.float32)
    return q, k, v, kr, ks, O.cu_seqlens_from_lengths(lens)


def _split(x, cu):
    return [x[cu[b]:cu[b + 1]] for b in range(len(cu) - 1)]


def test_rope_fp8_prefill_matches_bruteforce_on_torch_decoded_codes():
    lens = [3, 70, 130]
    q, k, v, kr, ks, cu = _case(81, lens, 4, 2, 8, 4, 6)
    out, lse = O.ragged_prefill_rope_fp8(q, k, v, kr, ks, cu, 0.29)
    krd = _t8(kr)[:, 0, :] * ks.astype(np.float64)[:, None]
    bo, bl = BF.prefill(_split(_tb(q), cu), _split(_tb(k), cu), _split(_tb(v), cu), lens, 0.29,
                        k_rope=_split(krd, cu))
    np.testing.assert_allclose(out, np.concatenate([np.array(x) for x in bo]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, np.concatenate([np.array(x) for x in bl]), rtol=0, atol=1e-12)


def test_rope_fp8_prefill_matches_sdpa_with_concatenated_rope_key():
    lens = [64, 100, 1, 150]
    sc = 1 / math.sqrt(24)
    q, k, v, kr, ks, cu = _case(82, lens, 4, 4, 16, 8, 16)
    out, _ = O.ragged_prefill_rope_fp8(q, k, v, kr, ks, cu, sc)
    ref = []
    for b in range(len(lens)):
        s = slice(cu[b], cu[b + 1])
        krd = _t8(kr[s]) * ks[s].astype(np.float64)[:, None, None]
        Q = _tb(q[s]).transpose(1, 0, 2)
        K = np.concatenate([_tb(k[s]), np.broadcast_to(krd, (lens[b], 4, 8))], axis=2).transpose(1, 0, 2)
        V = _tb(v[s]).transpose(1, 0, 2)
        o = F.scaled_dot_product_attention(torch.from_numpy(np.ascontiguousarray(Q)),
                                           torch.from_numpy(np.ascontiguousarray(K)),
                                           torch.from_numpy(np.ascontiguousarray(V)), is_causal=True, scale=sc)
        ref.append(o.numpy().transpose(1, 0, 2))
    np.testing.assert_allclose(out, np.concatenate(ref), rtol=0, atol=1e-10)


def test_rope_fp8_scales_touch_only_the_rope_term():
    """With a zero rope query the rope term vanishes: the result is plain
    attention on the per-head parts and does not depend on the rope scales
    (a scale applied to the whole score, or to the per-head part, would change
    it)."""
    lens = [70, 33]
    q, k, v, kr, ks, cu = _case(83, lens, 4, 4, 16, 8, 8)
    q = q.copy()
    q[:, :, 16:] = 0
    a = O.ragged_prefill_rope_fp8(q, k, v, kr, ks, cu, 0.3)
    b = O.ragged_prefill_rope_fp8(q, k, v, kr, (ks * 37.0).astype(np.float32), cu, 0.3)
    np.testing.assert_array_equal(a[0], b[0])
    bo, _ = BF.prefill(_split(_tb(q)[:, :, :16], cu), _split(_tb(k), cu), _split(_tb(v), cu), lens, 0.3)
    np.testing.assert_allclose(a[0], np.concatenate([np.array(x) for x in bo]), rtol=0, atol=1e-12)


def test_rope_fp8_with_power_of_two_scales_is_a_bf16_rope_key():
    """Codes times a power of two are exact bf16 values: the quantised form
    then equals the bf16 MLA prefill whose rope key holds those values (built
    with torch's casts), exactly."""
    lens = [90, 40, 5]
    q, k, v, kr, _, cu = _case(84, lens, 4, 2, 16, 8, 8)
    rng = np.random.default_rng(5)
    ks = (2.0 ** rng.integers(-9, -3, size=sum(lens))).astype(np.float32)
    krb = (torch.from_numpy(kr).view(torch.float8_e4m3fn).float() * torch.from_numpy(ks)[:, None, None])
    krb = krb.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    a = O.ragged_prefill_rope_fp8(q, k, v, kr, ks, cu, 0.21)
    b = O.ragged_prefill(q, k, v, cu, 0.21, k_rope=krb, dtype="bf16")
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_rope_fp8_zero_scale_acts_as_zero_codes_row_by_row():
    """A zero scale on a set of rows equals zero codes on exactly those rows:
    each scale belongs to its own token's rope row."""
    lens = [80, 61]
    q, k, v, kr, ks, cu = _case(85, lens, 2, 2, 16, 8, 8)
    rows = np.random.default_rng(6).choice(sum(lens), size=40, replace=False)
    ks0 = ks.copy()
    ks0[rows] = 0
    kr0 = kr.copy()
    kr0[rows] = 0
    a = O.ragged_prefill_rope_fp8(q, k, v, kr, ks0, cu, 0.25)
    b = O.ragged_prefill_rope_fp8(q, k, v, kr0, ks, cu, 0.25)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_rope_fp8_generator_recipe():
    """The generated case is the bf16 MLA case of the same seed with each rope
    row quantised at amax / 448 of the row, q, k and v unchanged."""
    c = gen.make_prefill_rope_fp8_case(name="r", seed=86, seq_lens=[40, 9], Hq=4, Hk=2)
    b = gen.make_prefill_case(name="r", seed=86, seq_lens=[40, 9], Hq=4, Hk=2, D_qk=192, D_rope=64, D_v=128)
    assert c.rope_dtype == "e4m3fn" and c.k_rope.dtype == np.uint8 and c.k_rope_scale.shape == (49,)
    for x, y in ((c.q, b.q), (c.k, b.k), (c.v, b.v)):
        np.testing.assert_array_equal(x, y)
    x = torch.from_numpy(b.k_rope.view(np.int16)).view(torch.bfloat16).float()
    amax = x.abs().amax(dim=(1, 2))
    want_sc = (amax / 448.0).numpy().astype(np.float32)
    np.testing.assert_array_equal(c.k_rope_scale, want_sc)
    want = (x / torch.from_numpy(want_sc)[:, None, None]).clamp(-448, 448).to(torch.float8_e4m3fn)
    np.testing.assert_array_equal(c.k_rope, want.view(torch.uint8).numpy())
