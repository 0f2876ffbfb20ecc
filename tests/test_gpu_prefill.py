"""Ragged causal prefill on the GPU through the C ABI, against the fp64 oracle.

bf16 inputs: max-abs-err of out against the oracle run on the same rounded
inputs must stay within 2e-2.  The LSE is fp32 from end to end and is held to
1e-3: one 64-key tile dropped from a row of a few thousand keys moves it by
about 1e-2.  The two full-size workloads are compared on every row and head."""
import numpy as np
import pytest
import torch

from oracle import attention as O
from oracle import parallel as OR
from workloads import gen

pytestmark = pytest.mark.gpu

TOL = 2e-2
LSE_TOL = 1e-3


@pytest.fixture(scope="module")
def gu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from tests import gpu_util  # imports the HIP library; fails loudly if it is missing
    return gpu_util


def _rows_sample(case, n_mid=64, seed=0):
    """First and last rows of each sequence, rows around 64/128 boundaries, random rows."""
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


def _check(gu, case, rows=None, tol=TOL):
    gu.announce(f"prefill {case.name} lens={list(case.seq_lens)[:8]} Hq={case.Hq} Hk={case.Hk} "
                f"Dqk={case.D_qk} Dr={case.D_rope} mask={case.block_mask is not None} seed={case.meta.get('seed')}")
    dp = gu.DevicePrefill(case)
    dp.run()
    out, lse = dp.results()
    ref_fn = lambda rr: O.ragged_prefill(case.q, case.k, case.v, case.cu_seqlens, case.scale,  # noqa: E731
                                         k_rope=case.k_rope, block_mask=case.block_mask, dtype="bf16", rows=rr)
    if rows is None:
        ref, ref_lse = OR.all_rows(ref_fn, case.T)
    else:
        ref, ref_lse = ref_fn(rows)
        out, lse = out[rows], lse[rows]
    e_out = gu.max_abs_err(out, ref)
    e_lse = gu.lse_err(lse, ref_lse)
    gu.announce(f"  max-abs-err out {e_out:.3e} lse {e_lse:.3e} (tol {tol:g}, lse {LSE_TOL:g}) "
                f"rows={'all' if rows is None else len(rows)}")
    assert e_out <= tol and e_lse <= LSE_TOL, (e_out, e_lse)
    return dp, out, lse


def test_prefill_mla_config_full_size(gu):
    """Every row and head of the ragged MLA workload (6584 tokens, 16 heads)."""
    _check(gu, gen.prefill_mla_bf16())


@pytest.mark.parametrize("mask", [None, 0.3])
def test_prefill_many_query_tile_indices(gu, mask):
    """Grids with more than 32 query-tile indices, where the kernel finds a
    workgroup's item by counting, in parallel over tile indices, the items at
    or past each: ragged lengths with an empty sequence and one of 4500 rows
    (36 tile indices of 128 rows; 71 of 64 rows with a mask and head pairs).
    Every row and head compared."""
    case = gen.make_prefill_case(name=f"many_tiles_{mask}", seed=91, seq_lens=[4500, 0, 2100, 130], Hq=8, Hk=2,
                                 D_qk=128, D_rope=0, D_v=128, mask_density=mask)
    _check(gu, case)


def test_prefill_blocksparse_config_full_size(gu):
    """Every row and head of the block-sparse workload (2 x 8192 tokens, 32
    query heads): every query tile and head pair the grid ranks is checked."""
    _check(gu, gen.prefill_blocksparse_bf16())


@pytest.mark.parametrize("rope", [0, 64])
def test_prefill_ragged_small(gu, rope):
    case = gen.make_prefill_case(name=f"ragged_r{rope}", seed=200 + rope, seq_lens=[1, 63, 64, 65, 130, 300, 7],
                                 Hq=8, Hk=8 if rope else 2, D_qk=128 + rope, D_rope=rope, D_v=128)
    _check(gu, case)


@pytest.mark.parametrize("Hq,Hk,rope", [(4, 2, 0), (16, 2, 0), (8, 4, 64)])
def test_prefill_head_pairs_with_mask_ragged(gu, Hq, Hk, rope):
    """A block mask with an even head ratio: each workgroup takes 64 rows of
    two heads of one KV group.  Sequences shorter than one wave's 32 rows,
    ends on and off the 32- and 64-row edges, and a mask of density 0.3."""
    case = gen.make_prefill_case(name=f"pairs_{Hq}_{Hk}_r{rope}", seed=240 + Hq + rope,
                                 seq_lens=[1, 2, 31, 33, 63, 64, 65, 97, 200, 513], Hq=Hq, Hk=Hk, D_qk=128 + rope,
                                 D_rope=rope, D_v=128, mask_density=0.3)
    dp, _, _ = _check(gu, case)
    assert dp.plan.q_tile_rows == 64


def test_prefill_gqa_ratios(gu):
    for Hq, Hk in ((8, 1), (16, 4), (4, 4)):
        case = gen.make_prefill_case(name=f"gqa_{Hq}_{Hk}", seed=210 + Hq, seq_lens=[200, 129], Hq=Hq, Hk=Hk,
                                     D_qk=128, D_rope=0, D_v=128)
        _check(gu, case)


def test_prefill_block_mask_small_with_hidden_diagonal(gu):
    case = gen.make_prefill_case(name="mask_small", seed=220, seq_lens=[300, 200], Hq=8, Hk=2, D_qk=128,
                                 D_rope=0, D_v=128, mask_density=0.4)
    m = case.block_mask.copy()
    m[0, 2, :] = 0            # query block 2 of sequence 0 sees nothing: its rows are 0 with lse -inf
    m[1, 1, 1] = 0            # diagonal off, first column still on
    case = gen.PrefillCase(**{**case.__dict__, "block_mask": m})
    dp, out, lse = _check(gu, case)
    assert np.all(out[128:192] == 0) and np.all(np.isneginf(lse[128:192]))


def test_prefill_all_on_mask_equals_dense(gu):
    case = gen.make_prefill_case(name="dense", seed=230, seq_lens=[257, 190], Hq=8, Hk=2, D_qk=192, D_rope=64,
                                 D_v=128)
    gu.announce("prefill all-on mask vs dense")
    a = gu.DevicePrefill(case)
    a.run()
    out1, lse1 = a.results()
    nb = (int(case.seq_lens.max()) + 63) // 64
    ones = np.tril(np.ones((case.B, nb, nb), np.uint8))
    case2 = gen.PrefillCase(**{**case.__dict__, "block_mask": ones})
    b = gu.DevicePrefill(case2)
    b.run()
    out2, lse2 = b.results()
    assert np.array_equal(out1, out2) and np.array_equal(lse1, lse2)


def test_prefill_first_row_is_its_value_row(gu):
    case = gen.make_prefill_case(name="first_row", seed=240, seq_lens=[5, 1, 70], Hq=4, Hk=4, D_qk=192,
                                 D_rope=64, D_v=128)
    gu.announce("prefill first rows")
    dp = gu.DevicePrefill(case)
    dp.run()
    out, _ = dp.results()
    for b in range(case.B):
        c0 = int(case.cu_seqlens[b])
        for h in range(case.Hq):
            assert np.array_equal(out[c0, h], O.widen(case.v[c0, h], "bf16")), (b, h)


def test_prefill_packed_equals_separate(gu):
    case = gen.make_prefill_case(name="packed", seed=250, seq_lens=[100, 333, 64], Hq=8, Hk=2, D_qk=128,
                                 D_rope=0, D_v=128)
    gu.announce("prefill packed vs separate")
    dp = gu.DevicePrefill(case)
    dp.run()
    out, _ = dp.results()
    for b in range(case.B):
        c0, c1 = int(case.cu_seqlens[b]), int(case.cu_seqlens[b + 1])
        sub = gen.PrefillCase(**{**case.__dict__, "seq_lens": case.seq_lens[b:b + 1],
                                 "cu_seqlens": np.array([0, c1 - c0], np.int32), "q": case.q[c0:c1],
                                 "k": case.k[c0:c1], "v": case.v[c0:c1]})
        sp = gu.DevicePrefill(sub)
        sp.run()
        o1, _ = sp.results()
        assert np.array_equal(o1, out[c0:c1]), b


def test_prefill_more_than_64_sequences(gu):
    """Batches above 64 sequences take the plain (sequence, query tile) grid order."""
    rng = np.random.default_rng(260)
    lens = rng.integers(0, 300, size=70).tolist()
    lens[:6] = [0, 1, 128, 129, 257, 64]
    case = gen.make_prefill_case(name="b70", seed=260, seq_lens=lens, Hq=4, Hk=2, D_qk=128, D_rope=0, D_v=128)
    _check(gu, case)


def test_prefill_more_than_64_sequences_with_mask(gu):
    rng = np.random.default_rng(261)
    lens = rng.integers(1, 400, size=66).tolist()
    case = gen.make_prefill_case(name="b66_mask", seed=261, seq_lens=lens, Hq=2, Hk=1, D_qk=192, D_rope=64,
                                 D_v=128, mask_density=0.4)
    _check(gu, case)


def test_prefill_empty_sequences_in_the_batch(gu):
    case = gen.make_prefill_case(name="empties", seed=262, seq_lens=[0, 5, 0, 200, 0, 129], Hq=4, Hk=4, D_qk=192,
                                 D_rope=64, D_v=128)
    _check(gu, case)


def test_prefill_single_long_sequence_sampled(gu):
    case = gen.make_prefill_case(name="long1", seed=263, seq_lens=[5000], Hq=2, Hk=1, D_qk=192, D_rope=64, D_v=128)
    _check(gu, case, rows=_rows_sample(case, n_mid=96))


def test_prefill_32k_sequence_sampled(gu):
    """A 32768-token MLA sequence: 256 query tiles, 512 key tiles (eight 64-tile
    schedule words), sampled rows checked one by one against the oracle."""
    case = gen.make_prefill_case(name="long32k", seed=264, seq_lens=[32768, 77], Hq=2, Hk=1, D_qk=192, D_rope=64,
                                 D_v=128)
    _check(gu, case, rows=_rows_sample(case, n_mid=48))


def test_prefill_32k_block_sparse_sampled(gu):
    case = gen.make_prefill_case(name="long32k_mask", seed=265, seq_lens=[32768], Hq=2, Hk=2, D_qk=128, D_rope=0,
                                 D_v=128, mask_density=0.1)
    _check(gu, case, rows=_rows_sample(case, n_mid=48))
