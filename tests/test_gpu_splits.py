"""Key-axis splits of the prefill kernels on the GPU: with num_splits forced
(and, for small grids, chosen by the plan) every prefill form matches the
fp64 oracle, and the split result equals the unsplit one up to rounding.
Cases include more splits than a short sequence has key tiles, so that some
splits see no key at all and write an empty partial."""
import numpy as np
import pytest
import torch

from oracle import attention as O
from oracle import parallel as OR
from tests.test_gpu_prefill_fp8 import fp8_lse_bound
from workloads import gen

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "e4m3fn": 6e-2}
LSE_TOL = 1e-3


@pytest.fixture(scope="module")
def gu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from tests import gpu_util  # imports the HIP library; fails loudly if it is missing
    return gpu_util


def _prefill_ref(case):
    if case.dtype == "e4m3fn":
        return O.ragged_prefill_fp8(case.q, case.q_rope, case.k, case.v, case.k_rope, case.cu_seqlens, case.scale,
                                    case.q_scale, case.k_scale, block_mask=case.block_mask)
    return O.ragged_prefill(case.q, case.k, case.v, case.cu_seqlens, case.scale, k_rope=case.k_rope,
                            block_mask=case.block_mask, dtype="bf16")


def _run_prefill(gu, case, ns):
    dp = gu.DevicePrefill(case, num_splits=ns)
    assert dp.plan.num_splits == ns
    dp.run()
    return dp.results()


def _check_prefill(gu, case, splits):
    ref, ref_lse = _prefill_ref(case)
    tol = TOL[case.dtype]
    base = None
    for ns in splits:
        gu.announce(f"split prefill {case.name} lens={list(case.seq_lens)[:6]} splits={ns}")
        out, lse = _run_prefill(gu, case, ns)
        e_out, e_lse = gu.max_abs_err(out, ref), gu.lse_err(lse, ref_lse)
        gu.announce(f"  max-abs-err out {e_out:.3e} lse {e_lse:.3e} (tol {tol:g})")
        # fp8 Q.K: the fp32 summation bound of the scores (see test_gpu_prefill_fp8)
        bound = fp8_lse_bound(case) if case.dtype == "e4m3fn" else LSE_TOL
        assert e_out <= tol and gu.lse_within(lse, ref_lse, bound), (ns, e_out, e_lse)
        if base is None:
            base = (out, lse)
        else:  # against the first (unsplit) run
            assert gu.max_abs_err(out, base[0]) <= 1e-2 and gu.lse_err(lse, base[1]) <= 1e-4


def test_split_ragged_mla(gu):
    case = gen.make_prefill_case(name="split_mla", seed=300, seq_lens=[1, 70, 700, 1500, 0, 129], Hq=8, Hk=8,
                                 D_qk=192, D_rope=64, D_v=128)
    _check_prefill(gu, case, (1, 2, 3, 4, 6))


@pytest.mark.parametrize("B", [63, 64, 65])
def test_split_many_sequences(gu, B):
    """The merge finds a row's sequence from lane-held bounds below 64
    sequences and by binary search from 64 on: batches on both sides of that
    edge, with empty and one-row sequences among them."""
    rng = np.random.default_rng(310 + B)
    lens = [int(x) for x in rng.integers(0, 140, size=B)]
    lens[0], lens[-1], lens[B // 2] = 0, 1, 129
    case = gen.make_prefill_case(name=f"split_b{B}", seed=310 + B, seq_lens=lens, Hq=4, Hk=2, D_qk=128, D_rope=0,
                                 D_v=128)
    _check_prefill(gu, case, (1, 2))


def test_split_merge_odd_pair_count(gu):
    """Above 16384 (row, head) pairs a merge wave takes two pairs: an odd
    count (5463 rows of 3 heads) leaves the last wave one pair past the end."""
    case = gen.make_prefill_case(name="split_odd", seed=320, seq_lens=[683] * 7 + [682], Hq=3, Hk=1, D_qk=128,
                                 D_rope=0, D_v=128)
    assert case.T * 3 == 16389
    _check_prefill(gu, case, (1, 2, 3))


def test_split_ragged_gqa_with_block_mask(gu):
    case = gen.make_prefill_case(name="split_mask", seed=301, seq_lens=[1100, 333, 64], Hq=8, Hk=2, D_qk=128,
                                 D_rope=0, D_v=128, mask_density=0.3)
    _check_prefill(gu, case, (1, 3))


@pytest.mark.parametrize("blockwise", [False, True])
def test_split_fp8(gu, blockwise):
    case = gen.make_prefill_fp8_case(name="split_fp8", seed=302, seq_lens=[900, 65, 300], Hq=8, Hk=2, D_rope=64,
                                     blockwise=blockwise)
    _check_prefill(gu, case, (1, 2))


@pytest.mark.parametrize("Dr", [0, 64])
def test_split_chunk(gu, Dr):
    case = gen.make_chunk_case(name="split_chunk", seed=303 + Dr, prefix_lens=[3000, 10, 700], q_lens=[200, 64, 5],
                               Hq=8, Hk=2 if Dr == 0 else 8, D_rope=Dr)
    kp_ref = None
    base = None
    for ns in (1, 2, 4):
        gu.announce(f"split chunk Dr={Dr} splits={ns}")
        dc = gu.DeviceChunk(case, num_splits=ns)
        assert dc.plan.num_splits == ns
        dc.append()
        dc.run()
        out, lse = dc.results()
        if kp_ref is None:
            pools = dc.pools_bits()
            want = O.append_kv(case.k_new, case.v_new, case.k_pool, case.v_pool, case.block_table,
                               case.cu_seqlens_q, case.kv_lens, kr_new=case.kr_new, kr_pool=case.kr_pool)
            assert len(pools) == len(want) and all(np.array_equal(g, r) for g, r in zip(pools, want)), \
                "appended pools differ from the oracle's"
            kp_ref = pools
            ref, ref_lse = O.chunk_prefill(case.q, pools[0], pools[1], case.block_table, case.cu_seqlens_q,
                                           case.kv_lens, case.scale, dtype="bf16",
                                           kr_pool=pools[2] if len(pools) == 3 else None)
            base = (out, lse)
        e_out, e_lse = gu.max_abs_err(out, ref), gu.lse_err(lse, ref_lse)
        gu.announce(f"  max-abs-err out {e_out:.3e} lse {e_lse:.3e}")
        assert e_out <= 2e-2 and e_lse <= LSE_TOL
        assert gu.max_abs_err(out, base[0]) <= 1e-2 and gu.lse_err(lse, base[1]) <= 1e-4


def test_split_chosen_by_the_plan_for_a_long_context_chunk(gu):
    """The long-context MLA chunk workload (one sequence, 64 workgroups) gets
    four splits from the plan; every row and head matches the oracle."""
    case = gen.prefill_chunk_long_mla_bf16()
    dc = gu.DeviceChunk(case)
    assert dc.plan.num_splits == 4
    dc.append()
    dc.run()
    out, lse = dc.results()
    pools = dc.pools_bits()
    want = O.append_kv(case.k_new, case.v_new, case.k_pool, case.v_pool, case.block_table, case.cu_seqlens_q,
                       case.kv_lens, kr_new=case.kr_new, kr_pool=case.kr_pool)
    assert len(pools) == len(want) and all(np.array_equal(g, r) for g, r in zip(pools, want)), \
        "appended pools differ from the oracle's"
    ref, ref_lse = OR.all_rows(lambda rr: O.chunk_prefill(case.q, pools[0], pools[1], case.block_table,
                                                          case.cu_seqlens_q, case.kv_lens, case.scale, dtype="bf16",
                                                          rows=rr, kr_pool=pools[2]), case.T, block=32)
    e_out, e_lse = gu.max_abs_err(out, ref), gu.lse_err(lse, ref_lse)
    gu.announce(f"long-context mla chunk, auto split: max-abs-err out {e_out:.3e} lse {e_lse:.3e}")
    assert e_out <= 2e-2 and e_lse <= LSE_TOL
