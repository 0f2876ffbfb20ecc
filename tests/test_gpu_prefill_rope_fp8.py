"""MLA prefill with a quantised shared rope key on the GPU, through the C ABI
(gqap_prefill_rope_fp8), against the fp64 oracle on the same codes, scales and
bf16 values.

The rope rows are e4m3fn codes with one scale per row; q, k and v are bf16.
Bar: max-abs-err of out within 6e-2 (fp8 inputs), the fp32 LSE within 1e-3;
the full-size workload is compared on every row and head.  With power-of-two
scales the codes times their scales are exact bf16 values, so the result must
match the bf16 prefill on those values up to the order of the fp32 sums."""
import numpy as np
import pytest
import torch

from oracle import attention as O
from oracle import parallel as OR
from workloads import gen

pytestmark = pytest.mark.gpu

TOL = 6e-2
LSE_TOL = 1e-3


@pytest.fixture(scope="module")
def gu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from tests import gpu_util  # imports the HIP library; fails loudly if it is missing
    return gpu_util


def _check(gu, case, num_splits=0):
    gu.announce(f"fp8-rope prefill {case.name} lens={list(case.seq_lens)[:8]} Hq={case.Hq} Hk={case.Hk} "
                f"mask={case.block_mask is not None} splits={num_splits} seed={case.meta.get('seed')}")
    dp = gu.DevicePrefill(case, num_splits=num_splits)
    assert dp.rope8
    dp.out.fill_(float("nan"))
    dp.run()
    out, lse = dp.results()
    ref_fn = lambda rr: O.ragged_prefill_rope_fp8(case.q, case.k, case.v, case.k_rope, case.k_rope_scale,  # noqa
                                                  case.cu_seqlens, case.scale, block_mask=case.block_mask, rows=rr)
    ref, ref_lse = OR.all_rows(ref_fn, case.T)
    e_out, e_lse = gu.max_abs_err(out, ref), gu.lse_err(lse, ref_lse)
    gu.announce(f"  max-abs-err out {e_out:.3e} lse {e_lse:.3e} (tol {TOL:g}, lse {LSE_TOL:g})")
    assert e_out <= TOL and e_lse <= LSE_TOL, (e_out, e_lse)
    return out, lse


def test_rope_fp8_config_full_size(gu):
    """Every row and head of the MLA workload with the rope key quantised per row."""
    _check(gu, gen.prefill_mla_rope_fp8())


@pytest.mark.parametrize("Hq,Hk", [(16, 16), (8, 2)])
def test_rope_fp8_small_ragged(gu, Hq, Hk):
    case = gen.make_prefill_rope_fp8_case(name="rope8_small", seed=91, seq_lens=[1, 63, 64, 65, 130, 300, 0, 7],
                                          Hq=Hq, Hk=Hk)
    _check(gu, case)


@pytest.mark.parametrize("Hq,Hk", [(8, 8), (8, 4)])
def test_rope_fp8_block_mask(gu, Hq, Hk):
    """A block mask (with an even head ratio the workgroups take head pairs)."""
    case = gen.make_prefill_rope_fp8_case(name="rope8_mask", seed=92, seq_lens=[333, 200, 64], Hq=Hq, Hk=Hk,
                                          mask_density=0.35)
    _check(gu, case)


def test_rope_fp8_key_axis_splits(gu):
    case = gen.make_prefill_rope_fp8_case(name="rope8_split", seed=93, seq_lens=[900, 65, 300], Hq=8, Hk=8)
    a, la = _check(gu, case, num_splits=1)
    b, lb = _check(gu, case, num_splits=3)
    assert gu.max_abs_err(a, b) <= 1e-2 and gu.lse_err(la, lb) <= 1e-4


def test_rope_fp8_with_power_of_two_scales_matches_the_bf16_prefill(gu):
    """Power-of-two row scales: the quantised rope key equals a bf16 rope key
    exactly, so the bf16 kernel on it gives the same result up to the order of
    the fp32 sums (rope first here, per-head part first there): a few bf16
    steps of the output (one step is 7.8e-3 at magnitudes in [1, 2)), 1e-4 on
    the fp32 LSE."""
    case = gen.make_prefill_rope_fp8_case(name="rope8_pow2", seed=94, seq_lens=[257, 190, 31], Hq=8, Hk=2)
    rng = np.random.default_rng(3)
    case.k_rope_scale = (2.0 ** rng.integers(-9, -4, size=case.T)).astype(np.float32)
    gu.announce("fp8-rope prefill with power-of-two scales vs the bf16 prefill")
    dp = gu.DevicePrefill(case)
    dp.run()
    out8, lse8 = dp.results()
    krb = (torch.from_numpy(case.k_rope).view(torch.float8_e4m3fn).float()
           * torch.from_numpy(case.k_rope_scale)[:, None, None]).to(torch.bfloat16)
    bf = gen.PrefillCase(**{**case.__dict__, "k_rope": krb.view(torch.int16).numpy().view(np.uint16),
                            "rope_dtype": "bf16", "k_rope_scale": None})
    db = gu.DevicePrefill(bf)
    db.run()
    outb, lseb = db.results()
    assert gu.max_abs_err(out8, outb) <= 2e-2 and gu.lse_err(lse8, lseb) <= 1e-4
