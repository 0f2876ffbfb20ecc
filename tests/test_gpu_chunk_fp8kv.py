"""Chunked prefill over an fp8 e4m3fn KV cache on the GPU, through the C ABI,
against the fp64 oracle.

gqap_append_kv_fp8 is byte work: it quantises the chunk's bf16 keys and values
with the per-tensor scales, and the pools after it must equal the oracle's
append bit for bit (a NaN input may give either NaN code: the sign of a NaN
carries nothing).  gqap_chunk_prefill_fp8kv reads the fp8 pages: max-abs-err
of out and lse against the oracle on the same codes stays within 6e-2, the
bound for fp8 KV.  At unit scales the fp8 path must give the bf16 path's bits
on a bf16 cache that holds the decoded codes (the widening is exact and the
math after it is shared).
"""
import dataclasses

import numpy as np
import pytest
import torch

from oracle import attention as O
from oracle import parallel as OR
from workloads import gen

pytestmark = pytest.mark.gpu

TOL = 6e-2
LSE_TOL = 1e-3   # the LSE is fp32 end to end


@pytest.fixture(scope="module")
def gu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from tests import gpu_util  # imports the HIP library; fails loudly if it is missing
    return gpu_util


def _oracle_pools(case):
    return O.append_kv(case.k_new, case.v_new, case.k_pool, case.v_pool, case.block_table, case.cu_seqlens_q,
                       case.kv_lens, kr_new=case.kr_new, kr_pool=case.kr_pool, kv_dtype="e4m3fn",
                       k_scale=case.k_scale, v_scale=case.v_scale)


def _codes_equal(got, ref):
    """Equal codes, except that a NaN code matches any NaN code."""
    nan_g = (got & 0x7F) == 0x7F
    nan_r = (ref & 0x7F) == 0x7F
    return np.array_equal(nan_g, nan_r) and np.array_equal(got[~nan_r], ref[~nan_r])


def _rows_sample(case, n_mid=48, seed=0):
    rng = np.random.default_rng(seed)
    rows = set()
    for b in range(case.B):
        c0, c1 = int(case.cu_seqlens_q[b]), int(case.cu_seqlens_q[b + 1])
        if c1 == c0:
            continue
        for r in (0, 1, 31, 32, 63, 64, 127, 128, 129):
            if c0 + r < c1:
                rows.add(c0 + r)
        rows.update({c1 - 1, c1 - 2} & set(range(c0, c1)))
        rows.update(rng.integers(c0, c1, size=min(n_mid, c1 - c0)).tolist())
    return np.array(sorted(rows), dtype=np.int64)


def _run(gu, case, rows=None, num_splits=0):
    gu.announce(f"fp8kv chunk {case.name} kv_lens={case.kv_lens.tolist()[:8]} q_lens={case.q_lens.tolist()[:8]} "
                f"Hq={case.Hq} Hk={case.Hk} Dr={case.D_rope} splits={num_splits} seed={case.meta.get('seed')}")
    dc = gu.DeviceChunk(case, num_splits=num_splits)
    dc.append()
    pools = _oracle_pools(case)
    got = dc.pools_bits()
    assert len(got) == len(pools)
    assert _codes_equal(got[0], pools[0]) and _codes_equal(got[1], pools[1]), "appended fp8 pools differ"
    if len(pools) == 3:
        assert np.array_equal(got[2], pools[2]), "appended rope pool differs"
    dc.run()
    out, lse = dc.results()
    ref_fn = lambda rr: O.chunk_prefill(case.q, pools[0], pools[1], case.block_table,  # noqa: E731
                                        case.cu_seqlens_q, case.kv_lens, case.scale, dtype="bf16", rows=rr,
                                        kr_pool=pools[2] if len(pools) == 3 else None, kv_dtype="e4m3fn",
                                        k_scale=case.k_scale, v_scale=case.v_scale)
    if rows is None:
        ref, ref_lse = OR.all_rows(ref_fn, case.T, block=128)
    else:
        ref, ref_lse = ref_fn(rows)
        out, lse = out[rows], lse[rows]
    e_out, e_lse = gu.max_abs_err(out, ref), gu.lse_err(lse, ref_lse)
    gu.announce(f"  max-abs-err out {e_out:.3e} lse {e_lse:.3e} (tol {TOL:g}, lse {LSE_TOL:g}) "
                f"rows={'all' if rows is None else len(rows)}")
    assert e_out <= TOL and e_lse <= LSE_TOL, (e_out, e_lse)
    return dc, out, lse


def test_fp8_append_quantises_every_bf16_value(gu):
    """The chunk's keys and values run through all 65536 bf16 bit patterns
    (zeros, subnormals, ties, values past the saturation point, infinities,
    NaNs), with a unit key scale and a fractional value scale; the written
    codes equal the oracle's quantiser bit for bit."""
    case = gen.make_chunk_case(name="fp8_append_all", seed=81, prefix_lens=[37], q_lens=[128], Hq=4, Hk=4,
                               kv_dtype="e4m3fn")
    pat = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).reshape(128, 4, 128)
    case = dataclasses.replace(case, k_new=pat, v_new=np.ascontiguousarray(pat[::-1]), k_scale=1.0,
                               v_scale=float(np.float32(0.0371)))
    gu.announce("fp8 append of every bf16 value")
    dc = gu.DeviceChunk(case)
    dc.append()
    got = dc.pools_bits()
    ref = _oracle_pools(case)
    assert _codes_equal(got[0], ref[0]) and _codes_equal(got[1], ref[1])
    # the rows outside the chunk are untouched (NaN codes of the generator)
    assert np.array_equal(got[0][~_written_mask(case)], case.k_pool[~_written_mask(case)])


def _written_mask(case):
    m = np.zeros(case.k_pool.shape, bool)
    for b in range(case.B):
        ql = int(case.q_lens[b])
        for i in range(ql):
            p = int(case.kv_lens[b]) - ql + i
            m[case.block_table[b, p // 64], :, p % 64, :] = True
    return m


def test_fp8kv_chunk_full_size(gu):
    """Every row and head of the chunked-prefill workload over the fp8 cache."""
    _run(gu, gen.prefill_chunk_fp8kv())


@pytest.mark.parametrize("Hq,Hk", [(8, 8), (8, 2), (16, 1)])
def test_fp8kv_chunk_small_ragged(gu, Hq, Hk):
    """Prefixes that start and end inside pages, chunks shorter and longer than
    a query tile, a chunk with no prefix."""
    case = gen.make_chunk_case(name="fp8kv_small", seed=82, prefix_lens=[0, 1, 63, 64, 100, 255, 700],
                               q_lens=[5, 64, 1, 130, 129, 200, 300], Hq=Hq, Hk=Hk, kv_dtype="e4m3fn")
    _run(gu, case)


def test_fp8kv_chunk_empty_and_one_token_chunks(gu):
    case = gen.make_chunk_case(name="fp8kv_edges", seed=83, prefix_lens=[10, 0, 500, 64, 3],
                               q_lens=[0, 1, 1, 0, 257], Hq=8, Hk=2, kv_dtype="e4m3fn")
    _run(gu, case)


@pytest.mark.parametrize("Hq,Hk", [(16, 16), (8, 2)])
def test_fp8kv_mla_chunk(gu, Hq, Hk):
    """MLA: the rope cache stays bf16, K nope and V pages are fp8."""
    case = gen.make_chunk_case(name="fp8kv_mla", seed=84, prefix_lens=[0, 63, 130, 700], q_lens=[5, 129, 64, 300],
                               Hq=Hq, Hk=Hk, D_rope=64, kv_dtype="e4m3fn")
    _run(gu, case)


@pytest.mark.parametrize("Dr", [0, 64])
def test_fp8kv_chunk_key_axis_splits(gu, Dr):
    """A long prefix with forced key-axis splits (partials merged by LSE)."""
    case = gen.make_chunk_case(name="fp8kv_split", seed=85 + Dr, prefix_lens=[3000, 17], q_lens=[200, 50], Hq=8,
                               Hk=2, D_rope=Dr, kv_dtype="e4m3fn")
    _run(gu, case, num_splits=3)


def test_fp8kv_long_prefix_sampled(gu):
    """A 9000-key cache (two 64-entry block-table words) and a 600-token chunk."""
    case = gen.make_chunk_case(name="fp8kv_long", seed=87, prefix_lens=[8400, 40], q_lens=[600, 40], Hq=8, Hk=1,
                               kv_dtype="e4m3fn")
    _run(gu, case, rows=_rows_sample(case))


@pytest.mark.parametrize("Dr", [0, 64])
def test_fp8kv_at_unit_scales_matches_bf16_cache_bits(gu, Dr):
    """Codes read with k_scale = v_scale = 1 give, bit for bit, the result of
    the bf16 path over a bf16 cache holding the decoded codes."""
    case = gen.make_chunk_case(name="fp8kv_bits", seed=88 + Dr, prefix_lens=[70, 0, 300], q_lens=[60, 130, 200],
                               Hq=8, Hk=2, D_rope=Dr, kv_dtype="e4m3fn")
    gu.announce(f"fp8kv vs bf16 cache bits Dr={Dr}")
    d8 = gu.DeviceChunk(case)
    d8.append()
    pools = d8.pools_bits()
    unit = dataclasses.replace(case, k_pool=pools[0], v_pool=pools[1], k_scale=1.0, v_scale=1.0,
                               kr_pool=pools[2] if Dr else None)
    d8 = gu.DeviceChunk(unit)
    d8.run()
    out8, lse8 = d8.results()
    widen = lambda c: torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    bf = dataclasses.replace(unit, kv_dtype="bf16", k_pool=widen(pools[0]), v_pool=widen(pools[1]))
    d16 = gu.DeviceChunk(bf)
    d16.run()
    out16, lse16 = d16.results()
    assert np.array_equal(out8, out16) and np.array_equal(lse8, lse16)


def test_fp8_append_then_paged_decode_reads_the_same_cache(gu):
    """One-token chunks appended into an fp8 cache, then the fp8 paged decode
    over the same pools and scales: both paths share the cache format, and
    both match the oracle's decode over the appended codes."""
    case = gen.make_chunk_case(name="fp8kv_decode", seed=90, prefix_lens=[1023, 64, 5, 300, 0],
                               q_lens=[1, 1, 1, 1, 1], Hq=16, Hk=4, kv_dtype="e4m3fn")
    dc, out_c, lse_c = _run(gu, case)
    kp, vp = dc.pools_bits()
    ref, ref_lse = O.paged_decode(case.q, kp, vp, case.block_table, case.kv_lens, case.scale, q_dtype="bf16",
                                  kv_dtype="e4m3fn", k_scale=case.k_scale, v_scale=case.v_scale)
    dec = dataclasses.make_dataclass("DecodeView", ["q", "k_pool", "v_pool", "block_table", "seq_lens", "q_dtype",
                                                     "kv_dtype", "scale", "k_scale", "v_scale", "B", "Hq"])
    view = dec(q=case.q, k_pool=kp, v_pool=vp, block_table=case.block_table, seq_lens=case.kv_lens, q_dtype="bf16",
               kv_dtype="e4m3fn", scale=case.scale, k_scale=case.k_scale, v_scale=case.v_scale, B=case.B, Hq=case.Hq)
    gu.announce("fp8 paged decode over the appended cache")
    dd = gu.DeviceDecode(view)
    dd.run()
    out_d, lse_d = dd.results()
    for out, lse in ((out_c, lse_c), (out_d, lse_d)):
        assert gu.max_abs_err(out, ref) <= TOL and gu.lse_err(lse, ref_lse) <= LSE_TOL


def test_fp8kv_long_context_mla_split_by_the_plan(gu):
    """One sequence with a 15872-token fp8 cache and a 512-token MLA chunk:
    64 workgroups, so the plan splits the key axis four ways; sampled rows
    (first, last, tile edges) match the oracle."""
    case = gen.make_chunk_case(name="fp8kv_long_mla", seed=91, prefix_lens=[15872], q_lens=[512], Hq=16, Hk=16,
                               D_rope=64, kv_dtype="e4m3fn")
    dc = gu.DeviceChunk(case)
    assert dc.plan.num_splits == 4
    _run(gu, case, rows=_rows_sample(case, n_mid=32))
