"""Pins for the oracle's fp8 KV cache in the chunked prefill: the e4m3fn
quantiser that the append writes with, the append into fp8 pages, and the
attention over them.  CPU only.

The quantiser is checked against torch's own float8_e4m3fn cast (round to
nearest even) over every bf16 value up to the saturation point, with two
scales, and against closed-form points (ties, subnormals, saturation, signed
zero); the attention against brute force on values decoded by torch."""
import numpy as np
import pytest
import torch

from oracle import attention as O
from oracle import bruteforce as BF
from workloads import gen


def _torch_codes(x32, scale):
    """torch's cast of x / scale (float32 division), after clamping to +-448
    (torch does not saturate: past 464 it gives NaN)."""
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)) / torch.tensor(np.float32(scale))
    return t.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _all_bf16_values():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    x = (bits.astype(np.uint32) << 16).view(np.float32)
    return x[np.isfinite(x)]


@pytest.mark.parametrize("scale", [1.0, 0.0371, 3.5])
def test_quantizer_matches_torch_cast_on_every_bf16_value(scale):
    x = _all_bf16_values()
    np.testing.assert_array_equal(O.quantize_e4m3fn(x, scale), _torch_codes(x, scale))


def test_quantizer_closed_form_points():
    pts = np.array([0.0, -0.0, 1.0, 1.0625, 1.1875, 448.0, 460.0, 464.0, 1e9, -1e9, 2.0 ** -10, 3 * 2.0 ** -10,
                    2.0 ** -9, 2.0 ** -6, 0.0146484375, -0.5], np.float32)
    want = [0x00, 0x80, 0x38, 0x38, 0x3A, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x00, 0x02, 0x01, 0x08, 0x08, 0xB0]
    # 1.0625 is halfway between 1.0 (0x38) and 1.125 (0x39): ties to the even 0x38;
    # 1.1875 between 1.125 and 1.25 goes to the even 0x3A; 2^-10 is half the
    # smallest subnormal (tie -> 0); 3*2^-10 between codes 1 and 2 -> 2;
    # 0.0146484375 = 7.5 * 2^-9 between the largest subnormal and 2^-6 -> 0x08
    np.testing.assert_array_equal(O.quantize_e4m3fn(pts, 1.0), np.array(want, np.uint8))
    nan = O.quantize_e4m3fn(np.array([np.nan, -np.nan], np.float32), 1.0)
    assert (nan[0] & 0x7F) == 0x7F and (nan[1] & 0x7F) == 0x7F


def test_quantizer_error_is_within_half_a_step():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(100000) * 3).astype(np.float32)
    sc = 0.013
    c = O.quantize_e4m3fn(x, sc)
    back = O.e4m3fn_to_f64(c) * sc
    a = np.abs(x.astype(np.float64))
    step = np.where(a / sc >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(a / sc, 2.0 ** -6))) - 3), 2.0 ** -9) * sc
    ok = a / sc <= 448
    assert np.all(np.abs(back - x)[ok] <= step[ok] / 2 * (1 + 1e-6))


def test_fp8_append_writes_quantized_codes_at_the_chunk_positions():
    """The fp8 append equals the bf16 append of the same tokens followed by
    quantisation of exactly the written rows; nothing else changes."""
    rng = np.random.default_rng(51)
    Hk, D, NB = 2, 8, 12
    kv_lens, q_lens = [70, 3, 128], [6, 3, 64]
    table = rng.permutation(NB)[:6].reshape(3, 2).astype(np.int32)
    kp = rng.integers(0, 0x7E, size=(NB, Hk, 64, D)).astype(np.uint8)
    vp = rng.integers(0, 0x7E, size=(NB, Hk, 64, D)).astype(np.uint8)
    cu = O.cu_seqlens_from_lengths(q_lens)
    kn = gen.to_bf16_bits(rng.standard_normal((int(cu[-1]), Hk, D)).astype(np.float32))
    vn = gen.to_bf16_bits(rng.standard_normal((int(cu[-1]), Hk, D)).astype(np.float32))
    ks, vs = 0.011, 0.02
    kp2, vp2 = O.append_kv(kn, vn, kp, vp, table, cu, np.array(kv_lens, np.int32), kv_dtype="e4m3fn",
                           k_scale=ks, v_scale=vs)
    kq = _torch_codes(O.bf16_to_f64(kn).astype(np.float32), ks)
    vq = _torch_codes(O.bf16_to_f64(vn).astype(np.float32), vs)
    kp3, vp3 = O.append_kv(kq, vq, kp, vp, table, cu, np.array(kv_lens, np.int32))
    np.testing.assert_array_equal(kp2, kp3)
    np.testing.assert_array_equal(vp2, vp3)
    assert not np.array_equal(kp2, kp)


def test_fp8_chunk_prefill_matches_bruteforce_on_torch_decoded_pages():
    rng = np.random.default_rng(52)
    Hq, Hk, D = 4, 2, 8
    kv_lens, q_lens = [70, 5, 130], [6, 5, 64]
    nblk = 3
    NB = 3 * nblk + 2
    table = rng.permutation(NB)[: 3 * nblk].reshape(3, nblk).astype(np.int32)
    kp = rng.integers(0, 0x7E, size=(NB, Hk, 64, D)).astype(np.uint8) | (rng.integers(0, 2, size=(NB, Hk, 64, D)).astype(np.uint8) << 7)
    vp = rng.integers(0, 0x7E, size=(NB, Hk, 64, D)).astype(np.uint8) | (rng.integers(0, 2, size=(NB, Hk, 64, D)).astype(np.uint8) << 7)
    cu = O.cu_seqlens_from_lengths(q_lens)
    q = rng.standard_normal((int(cu[-1]), Hq, D))
    ks, vs = 0.004, 0.01
    out, lse = O.chunk_prefill(q, kp, vp, table, cu, np.array(kv_lens, np.int32), 0.3, kv_dtype="e4m3fn",
                               k_scale=ks, v_scale=vs)
    dec = lambda c: torch.from_numpy(c).view(torch.float8_e4m3fn).double().numpy()
    K = [np.stack([dec(kp[table[b, t // 64], :, t % 64]) for t in range(L)]) * ks for b, L in enumerate(kv_lens)]
    V = [np.stack([dec(vp[table[b, t // 64], :, t % 64]) for t in range(L)]) * vs for b, L in enumerate(kv_lens)]
    qs = [q[cu[b]:cu[b + 1]] for b in range(3)]
    bo, bl = BF.chunk_prefill(qs, K, V, [kv_lens[b] - q_lens[b] for b in range(3)], 0.3)
    np.testing.assert_allclose(out, np.concatenate([np.array(x) for x in bo]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, np.concatenate([np.array(x) for x in bl]), rtol=0, atol=1e-12)
