"""fp8 ragged prefill on the GPU through the C ABI (gqap_prefill_fp8 and
gqap_prefill_fp8_blockwise), against the fp64 oracle run on the same fp8 codes
and bf16 values.

The nope parts of Q and K are e4m3fn codes with one scale per tensor, or one
per row of a head; the rope parts and V are bf16.  Bar: max-abs-err of out
within 6e-2, the tolerance for fp8 inputs.  The fp32 LSE is held to 1e-3
plus the fp32 summation bound of its scores: the LSE moves by at most the
largest error of a score, and a score summed in fp32 from n exact products
errs by at most n * 2^-24 * (the sum of the products' magnitudes).  With
row scales spread over three decades the products of one score reach a few
hundred in magnitude and cancel, so the bound there is a few 1e-3; at the
workloads' scales it is about 1e-4, far below the 2e-2 shift of a dropped
key tile.  The two full-size workloads are compared on every row and head."""
import numpy as np
import pytest
import torch

from oracle import attention as O
from oracle import parallel as OR
from workloads import gen

pytestmark = pytest.mark.gpu

TOL = 6e-2
LSE_TOL = 1e-3


def fp8_lse_bound(case) -> np.ndarray:
    """[T, Hq]: 1e-3 plus (Dn + Dr) * 2^-24 * scale * max over the keys of
    the sequence of sum_d |q_d k_d| (dequantised nope parts and rope parts),
    the fp32 summation bound of the row's largest score error."""
    qs, ks = np.asarray(case.q_scale, np.float64), np.asarray(case.k_scale, np.float64)
    qa = np.abs(O.widen(case.q, "e4m3fn") * (qs[..., None] if qs.ndim else qs))
    ka = np.abs(O.widen(case.k, "e4m3fn") * (ks[..., None] if ks.ndim else ks))
    n = case.D_nope + case.D_rope
    r = case.Hq // case.Hk
    bound = np.full((case.T, case.Hq), LSE_TOL)
    for b in range(case.B):
        c0, c1 = int(case.cu_seqlens[b]), int(case.cu_seqlens[b + 1])
        if c1 == c0:
            continue
        for h in range(case.Hq):
            m = qa[c0:c1, h] @ ka[c0:c1, h // r].T
            if case.D_rope:
                m = m + np.abs(O.widen(case.q_rope[c0:c1, h], "bf16")) @ np.abs(O.widen(case.k_rope[c0:c1, 0],
                                                                                        "bf16")).T
            bound[c0:c1, h] += n * 2.0 ** -24 * case.scale * m.max(axis=1)
    return bound


@pytest.fixture(scope="module")
def gu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from tests import gpu_util  # imports the HIP library; fails loudly if it is missing
    return gpu_util


def _rows_sample(case, n_mid=64, seed=0):
    rng = np.random.default_rng(seed)
    rows = set()
    for b in range(case.B):
        c0, c1 = int(case.cu_seqlens[b]), int(case.cu_seqlens[b + 1])
        if c1 == c0:
            continue
        for r in (0, 1, 31, 32, 63, 64, 65, 127, 128, 129):
            if c0 + r < c1:
                rows.add(c0 + r)
        rows.update({c1 - 1, c1 - 2, c1 - 64} & set(range(c0, c1)))
        rows.update(rng.integers(c0, c1, size=min(n_mid, c1 - c0)).tolist())
    return np.array(sorted(rows), dtype=np.int64)


def _sc(x):
    return f"per-row {np.shape(x)}" if np.ndim(x) else f"{x:.3g}"


def _check(gu, case, rows=None, tol=TOL):
    gu.announce(f"fp8 prefill {case.name} lens={list(case.seq_lens)[:8]} Hq={case.Hq} Hk={case.Hk} "
                f"Dr={case.D_rope} mask={case.block_mask is not None} qs={_sc(case.q_scale)} ks={_sc(case.k_scale)} "
                f"seed={case.meta.get('seed')}")
    dp = gu.DevicePrefill(case)
    dp.run()
    out, lse = dp.results()
    ref_fn = lambda rr: O.ragged_prefill_fp8(case.q, case.q_rope, case.k, case.v, case.k_rope,  # noqa: E731
                                             case.cu_seqlens, case.scale, case.q_scale, case.k_scale,
                                             block_mask=case.block_mask, rows=rr)
    if rows is None:
        ref, ref_lse = OR.all_rows(ref_fn, case.T)
    else:
        ref, ref_lse = ref_fn(rows)
        out, lse = out[rows], lse[rows]
    e_out = gu.max_abs_err(out, ref)
    e_lse = gu.lse_err(lse, ref_lse)
    bound = fp8_lse_bound(case)
    if rows is not None:
        bound = bound[rows]
    gu.announce(f"  max-abs-err out {e_out:.3e} lse {e_lse:.3e} (tol {tol:g}, lse bound {bound.max():.2e}) "
                f"rows={'all' if rows is None else len(rows)}")
    assert e_out <= tol and gu.lse_within(lse, ref_lse, bound), (e_out, e_lse)
    return dp, out, lse


def test_fp8_mla_config_full_size(gu):
    _check(gu, gen.prefill_mla_fp8())


@pytest.mark.parametrize("Hq,Hk", [(16, 16), (8, 2)])
def test_fp8_mla_small_ragged(gu, Hq, Hk):
    """Lengths inside one tile, on tile and 128-row boundaries, and past them."""
    case = gen.make_prefill_fp8_case(name="fp8_mla_small", seed=81, seq_lens=[1, 63, 64, 65, 130, 300], Hq=Hq,
                                     Hk=Hk, D_rope=64)
    _check(gu, case)


@pytest.mark.parametrize("Hq,Hk", [(8, 8), (16, 2)])
def test_fp8_without_rope(gu, Hq, Hk):
    """Plain GQA prefill with fp8 Q and K (the scales join the softmax constant)."""
    case = gen.make_prefill_fp8_case(name="fp8_gqa", seed=82, seq_lens=[5, 128, 257, 700], Hq=Hq, Hk=Hk, D_rope=0)
    _check(gu, case)


def test_fp8_block_mask(gu):
    case = gen.make_prefill_fp8_case(name="fp8_mask", seed=83, seq_lens=[900, 333], Hq=8, Hk=2, D_rope=64,
                                     mask_density=0.3)
    _check(gu, case)


def test_fp8_empty_and_single_token_sequences(gu):
    case = gen.make_prefill_fp8_case(name="fp8_edges", seed=84, seq_lens=[0, 1, 0, 2, 129], Hq=4, Hk=4, D_rope=64)
    _check(gu, case)


def test_fp8_zero_nope_codes_leave_rope_attention(gu):
    """All q_nope codes zero: the nope term vanishes, so the kernel must give
    rope-only attention whatever the two scales are (a scale applied to the
    whole score would change it)."""
    case = gen.make_prefill_fp8_case(name="fp8_zero_nope", seed=85, seq_lens=[200, 70], Hq=4, Hk=4, D_rope=64)
    case.q = np.zeros_like(case.q)
    case.q_scale, case.k_scale = 3.0, 5.0
    dp, out, lse = _check(gu, case)
    case.q_scale, case.k_scale = 0.01, 0.02
    dp2 = gu.DevicePrefill(case)
    dp2.run()
    out2, lse2 = dp2.results()
    np.testing.assert_array_equal(out, out2)
    np.testing.assert_array_equal(lse, lse2)


def test_fp8_long_sequence_sampled(gu):
    case = gen.make_prefill_fp8_case(name="fp8_long", seed=86, seq_lens=[8192], Hq=8, Hk=1, D_rope=64)
    _check(gu, case, rows=_rows_sample(case))


# ---------------------------------------------------------------- blockwise scales (gqap_prefill_fp8_blockwise)

def test_fp8_blockwise_mla_config_full_size(gu):
    _check(gu, gen.prefill_mla_fp8_blockwise())


@pytest.mark.parametrize("Hq,Hk,Dr", [(16, 16, 64), (8, 2, 64), (8, 2, 0), (4, 1, 0)])
def test_fp8_blockwise_small_ragged(gu, Hq, Hk, Dr):
    case = gen.make_prefill_fp8_case(name="fp8_bw_small", seed=87, seq_lens=[1, 63, 64, 65, 130, 300], Hq=Hq,
                                     Hk=Hk, D_rope=Dr, blockwise=True)
    _check(gu, case)


def test_fp8_blockwise_spread_scales_and_mask(gu):
    """Row scales spread over three decades (codes unchanged), so a scale taken
    from the wrong key, row or head shows; with a block mask and a ragged end."""
    case = gen.make_prefill_fp8_case(name="fp8_bw_spread", seed=88, seq_lens=[700, 333], Hq=8, Hk=2, D_rope=64,
                                     mask_density=0.4, blockwise=True)
    rng = np.random.default_rng(5)
    case.q_scale = (case.q_scale * 10.0 ** rng.uniform(-1.5, 1.0, size=case.q_scale.shape)).astype(np.float32)
    case.k_scale = (case.k_scale * 10.0 ** rng.uniform(-1.5, 1.0, size=case.k_scale.shape)).astype(np.float32)
    _check(gu, case)


def test_fp8_blockwise_equal_scales_match_per_tensor(gu):
    """Blockwise arrays that hold one value everywhere give the per-tensor
    kernel's result to within rounding of the order of the two multiplies."""
    case = gen.make_prefill_fp8_case(name="fp8_bw_eq", seed=89, seq_lens=[300, 129], Hq=8, Hk=2, D_rope=64)
    dp = gu.DevicePrefill(case)
    dp.run()
    out_t, lse_t = dp.results()
    T = case.T
    case.q_scale = np.full((T, case.Hq), case.q_scale, np.float32)
    case.k_scale = np.full((T, case.Hk), case.k_scale, np.float32)
    dpb = gu.DevicePrefill(case)
    assert dpb.blockwise
    dpb.run()
    out_b, lse_b = dpb.results()
    assert gu.max_abs_err(out_b, out_t) <= 1e-2 and gu.lse_err(lse_b, lse_t) <= 1e-4
