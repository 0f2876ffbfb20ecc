"""Short chunks on the paged-decode workers, on the GPU through the C ABI,
against the fp64 oracle's chunked prefill.

A chunk plan whose (token, query head) pairs of one KV head fit in as many
16-wide tiles as one token's heads (no forced splits) runs gqap_chunk_prefill
/ gqap_chunk_prefill_fp8kv on the decode workers (plan kernel 5, or 6 for an
fp8 cache), the MLA form (64-wide rope rows from the paged rope cache) on
their rope variant.  Every column of a tile is then one (token, head) pair
with its own causal key bound, kv_len - q_len + i for row i.  The
attention is the chunked prefill's, so the bars are the chunk tests': bf16
max-abs-err 2e-2, fp8 cache 6e-2, LSE 1e-3.  Pool rows past each sequence's
keys hold NaN, so a read past a row's keys shows up as NaN.
"""
import numpy as np
import pytest
import torch

from oracle import attention as O
from oracle import parallel as OR
from workloads import gen

pytestmark = pytest.mark.gpu

TOL = 2e-2
TOL_FP8 = 6e-2
LSE_TOL = 1e-3
NAN = float("nan")


@pytest.fixture(scope="module")
def gu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from tests import gpu_util  # imports the HIP library; fails loudly if it is missing
    return gpu_util


def _oracle_pools(case):
    fp8 = case.kv_dtype == "e4m3fn"
    return O.append_kv(case.k_new, case.v_new, case.k_pool, case.v_pool, case.block_table, case.cu_seqlens_q,
                       case.kv_lens, kr_new=case.kr_new, kr_pool=case.kr_pool,
                       kv_dtype=case.kv_dtype if fp8 else "bf16",
                       k_scale=case.k_scale if fp8 else 1.0, v_scale=case.v_scale if fp8 else 1.0)


def _oracle(case, pools, rows=None):
    fp8 = case.kv_dtype == "e4m3fn"
    kw = dict(kv_dtype="e4m3fn", k_scale=case.k_scale, v_scale=case.v_scale) if fp8 else {}
    kr = pools[2] if len(pools) == 3 else None
    fn = lambda rr: O.chunk_prefill(case.q, pools[0], pools[1], case.block_table, case.cu_seqlens_q,  # noqa: E731
                                    case.kv_lens, case.scale, dtype="bf16", rows=rr, kr_pool=kr, **kw)
    return OR.all_rows(fn, case.T, block=64) if rows is None else fn(rows)


def _run(gu, case, num_splits=0, want_kernel=None):
    fp8 = case.kv_dtype == "e4m3fn"
    gu.announce(f"short chunk {case.name} kv_lens={case.kv_lens.tolist()[:8]} q_lens={case.q_lens.tolist()[:8]} "
                f"Hq={case.Hq} Hk={case.Hk} kv={case.kv_dtype} splits={num_splits} seed={case.meta.get('seed')}")
    dc = gu.DeviceChunk(case, num_splits=num_splits)
    want = want_kernel if want_kernel is not None else (6 if fp8 else 5)
    assert dc.plan.kernel == want, (dc.plan.kernel, want)
    dc.out.fill_(NAN)
    dc.lse.fill_(NAN)
    dc.append()
    pools = _oracle_pools(case)
    got = dc.pools_bits()
    for g, r in zip(got, pools):
        if fp8 and g.dtype == np.uint8:   # a NaN input may give either NaN code
            nan_g, nan_r = (g & 0x7F) == 0x7F, (r & 0x7F) == 0x7F
            assert np.array_equal(nan_g, nan_r) and np.array_equal(g[~nan_r], r[~nan_r]), "appended pool differs"
        else:
            assert np.array_equal(g, r), "appended pool differs from the oracle's"
    dc.run()
    out, lse = dc.results()
    ref, ref_lse = _oracle(case, pools)
    tol = TOL_FP8 if fp8 else TOL
    e_out, e_lse = gu.max_abs_err(out, ref), gu.lse_err(lse, ref_lse)
    gu.announce(f"  kernel {dc.plan.kernel}: max-abs-err out {e_out:.3e} lse {e_lse:.3e} (tol {tol:g}, "
                f"lse {LSE_TOL:g})")
    assert e_out <= tol and e_lse <= LSE_TOL, (e_out, e_lse)
    return out, lse


@pytest.mark.parametrize("q_len", [1, 2, 4])
def test_multitoken_decode_full_size(gu, q_len):
    """Every row and head of the multi-token decode workload: 64 sequences of
    1024..4096 keys, 32 query heads on 8 KV heads, the last q_len keys the
    chunk's own."""
    _run(gu, gen.decode_multitoken(q_len))


@pytest.mark.parametrize("q_len", [1, 2])
def test_multitoken_mla_decode_full_size(gu, q_len):
    """Every row and head of the multi-token MLA decode: the same 64-sequence
    cache shape with 16 query heads, each its own KV head, and the 64-wide
    rope rows in the paged rope cache."""
    _run(gu, gen.decode_multitoken(q_len, Hq=16, Hk=16, D_rope=64))


# (Hq, Hk, longest chunk) with the rope cache
ROPE_SHAPES = [(16, 16, 4), (16, 16, 16), (8, 2, 4), (4, 1, 3)]


@pytest.mark.parametrize("Hq,Hk,qmax", ROPE_SHAPES)
def test_short_mla_chunks_ragged(gu, Hq, Hk, qmax):
    """The ragged lengths of the plain test below, with the rope part: prefixes
    on both sides of a page edge, empty chunks, a chunk that is its whole
    sequence, a sequence of more than 4096 keys."""
    prefix = [0, 1, 63, 64, 100, 255, 700, 4097, 62, 127]
    q_lens = [qmax, 1, qmax, 0, max(1, qmax - 1), qmax, 2 if qmax >= 2 else 1, qmax, qmax, 0]
    case = gen.make_chunk_case(name=f"short_mla_{Hq}x{Hk}_q{qmax}", seed=921 + Hq + Hk + qmax,
                               prefix_lens=prefix, q_lens=q_lens, Hq=Hq, Hk=Hk, D_rope=64)
    _run(gu, case)


def test_short_mla_chunks_fp8_cache(gu):
    """fp8 pages with the bf16 rope cache: k_scale multiplies the per-head sum
    only."""
    case = gen.make_chunk_case(name="short_mla_fp8", seed=931, prefix_lens=[0, 63, 64, 700, 2000, 5],
                               q_lens=[2, 2, 1, 2, 2, 0], Hq=16, Hk=16, D_rope=64, kv_dtype="e4m3fn")
    _run(gu, case)


# (Hq, Hk, longest chunk): one 16-column tile of 16, 15 or 12 pairs; ratio
# 32 with one token takes two tiles, as its decode does
SHAPES = [(8, 2, 4), (4, 4, 16), (16, 2, 2), (16, 1, 1), (32, 1, 1), (10, 2, 3), (12, 4, 5)]


@pytest.mark.parametrize("Hq,Hk,qmax", SHAPES)
def test_short_chunks_ragged(gu, Hq, Hk, qmax):
    """Prefixes that end on both sides of a page edge, chunks of every length
    up to the plan's, empty chunks, a chunk that is its whole sequence, and a
    sequence of more than 4096 keys.  With one-unit workers and causal bounds
    inside a page, some pieces end before a row's first masked key and some
    hold no key of a row at all."""
    prefix = [0, 1, 63, 64, 100, 255, 700, 4097, 62, 127]
    q_lens = [qmax, 1, qmax, 0, max(1, qmax - 1), qmax, 2 if qmax >= 2 else 1, qmax, qmax, 0]
    case = gen.make_chunk_case(name=f"short_{Hq}x{Hk}_q{qmax}", seed=901 + Hq + Hk + qmax, prefix_lens=prefix,
                               q_lens=q_lens, Hq=Hq, Hk=Hk)
    _run(gu, case)


def test_short_chunks_fp8_cache(gu):
    case = gen.make_chunk_case(name="short_fp8", seed=911, prefix_lens=[0, 63, 64, 700, 2000, 5],
                               q_lens=[4, 4, 1, 3, 4, 0], Hq=8, Hk=2, kv_dtype="e4m3fn")
    _run(gu, case)


def test_forced_splits_keep_the_prefill_kernel(gu):
    """num_splits = 1 keeps the prefill kernel for the same short chunks; both
    kernels meet the oracle."""
    case = gen.make_chunk_case(name="short_forced", seed=912, prefix_lens=[10, 300, 64, 1500],
                               q_lens=[4, 2, 4, 1], Hq=16, Hk=4)
    a, la = _run(gu, case)
    b, lb = _run(gu, case, num_splits=1, want_kernel=1)
    assert gu.max_abs_err(a, b) <= 2 * TOL


def test_short_chunks_past_the_capacity(gu):
    """Plan capacities max_q_len 4, max_kv_len 1000.  Chunk 0 (6 tokens)
    keeps its first 4 rows, computed with the whole chunk's causal offset,
    and its last 2 rows are 0 / -inf; chunk 2 has 1504 keys and chunk 3
    fewer keys than tokens: all their rows are 0 / -inf and neither is
    appended; chunk 1 is ordinary."""
    case = gen.make_chunk_case(name="short_cap", seed=913, prefix_lens=[100, 64, 1500, 3], q_lens=[6, 3, 4, 2],
                               Hq=8, Hk=2)
    case.kv_lens = case.kv_lens.copy()
    case.kv_lens[3] = 1                       # 2 tokens, 1 key
    gu.announce(f"short chunk capacity: kv_lens {case.kv_lens.tolist()} q_lens {case.q_lens.tolist()}")
    dc = gu.DeviceChunk(case, max_q_len=4, max_kv_len=1000, validate=False)
    assert dc.plan.kernel == 5
    dc.out.fill_(NAN)
    dc.lse.fill_(NAN)
    dc.append()
    kp, vp = dc.pools_bits()
    sub = gen.ChunkCase(**{**case.__dict__, "kv_lens": case.kv_lens[:2], "cu_seqlens_q": case.cu_seqlens_q[:3],
                           "block_table": case.block_table[:2]})
    want_k, want_v = O.append_kv(case.k_new, case.v_new, case.k_pool, case.v_pool, sub.block_table,
                                 sub.cu_seqlens_q, sub.kv_lens)
    assert np.array_equal(kp, want_k) and np.array_equal(vp, want_v), "append wrote outside the capacity"
    dc.run()
    out, lse = dc.results()
    cu = case.cu_seqlens_q
    cut = np.concatenate([np.arange(cu[0] + 4, cu[1]), np.arange(cu[2], cu[4])])
    assert np.all(out[cut] == 0) and np.all(np.isneginf(lse[cut]))
    keep = np.concatenate([np.arange(cu[0], cu[0] + 4), np.arange(cu[1], cu[2])])
    ref, ref_lse = O.chunk_prefill(case.q, want_k, want_v, case.block_table, case.cu_seqlens_q, case.kv_lens,
                                   case.scale, dtype="bf16", rows=keep)
    e_out, e_lse = gu.max_abs_err(out[keep], ref), gu.lse_err(lse[keep], ref_lse)
    gu.announce(f"  rows inside the capacity: out {e_out:.3e} lse {e_lse:.3e}")
    assert e_out <= TOL and e_lse <= LSE_TOL


def test_short_chunks_with_padded_strides(gu):
    """Strided q, out, chunk rows and pools on the decode workers; the
    padding reads NaN and the output padding stays NaN."""
    from tests.test_gpu_boundary import _padded, _padded_pool, _padding_untouched
    import gqa_attention_paged_amd as gq
    case = gen.make_chunk_case(name="short_strided", seed=914, prefix_lens=[0, 63, 300, 1000],
                               q_lens=[4, 3, 1, 4], Hq=8, Hk=2)
    gu.announce("short chunks, padded strides")
    dc = gu.DeviceChunk(case)
    dc.q = _padded(dc.q)
    dc.k_new, dc.v_new = _padded(dc.k_new, pad_mid=2), _padded(dc.v_new, pad_mid=2)
    dc.k_pool, dc.v_pool = _padded_pool(dc.k_pool), _padded_pool(dc.v_pool)
    dc.out = _padded(torch.empty_like(dc.out))
    dc.desc = gq.chunk_desc(dc.q, dc.k_new, dc.k_pool, dc.bt, batch=case.B, max_q_len=4,
                            max_kv_len=int(case.kv_lens.max()), out=dc.out)
    assert dc.desc.kv_stride_head > 64 * 128 and dc.desc.q_stride_token > case.Hq * 128
    dc.plan = gq.gqap_chunk_plan(dc.desc)
    assert dc.plan.kernel == 5
    dc.ws = torch.empty(dc.plan.workspace_bytes, dtype=torch.uint8, device=dc.q.device)
    dc.append()
    pools = _oracle_pools(case)
    dc.run()
    out, lse = dc.results()
    ref, ref_lse = _oracle(case, pools)
    assert gu.max_abs_err(out, ref) <= TOL and gu.lse_err(lse, ref_lse) <= LSE_TOL
    assert _padding_untouched(dc.out)
