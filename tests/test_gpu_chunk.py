"""Chunked prefill against a paged KV cache on the GPU, through the C ABI,
against the fp64 oracle.

gqap_append_kv is byte work: the pools after the append must equal the
oracle's append bit for bit.  gqap_chunk_prefill takes bf16 inputs: max-abs-err
of out and lse against the oracle on the same rounded inputs stays within 2e-2.
Every pool row that is not a key of its sequence (tails past kv_len, spare
blocks) holds NaN, so a read outside the keys shows up as NaN.
"""
import numpy as np
import pytest
import torch

from oracle import attention as O
from oracle import parallel as OR
from workloads import gen

pytestmark = pytest.mark.gpu

TOL = 2e-2
LSE_TOL = 1e-3   # the LSE is fp32 end to end; one dropped 64-key tile moves it by ~1e-2


@pytest.fixture(scope="module")
def gu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from tests import gpu_util  # imports the HIP library; fails loudly if it is missing
    return gpu_util


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


def _run(gu, case, rows=None, tol=TOL):
    gu.announce(f"chunk {case.name} kv_lens={case.kv_lens.tolist()[:8]} q_lens={case.q_lens.tolist()[:8]} "
                f"Hq={case.Hq} Hk={case.Hk} Dr={case.D_rope} seed={case.meta.get('seed')}")
    dc = gu.DeviceChunk(case)
    dc.append()
    pools = O.append_kv(case.k_new, case.v_new, case.k_pool, case.v_pool, case.block_table, case.cu_seqlens_q,
                        case.kv_lens, kr_new=case.kr_new, kr_pool=case.kr_pool)
    got = dc.pools_bits()
    assert len(got) == len(pools) and all(np.array_equal(g, r) for g, r in zip(got, pools)), \
        "appended pools differ from the oracle's"
    kp, vp = pools[0], pools[1]
    dc.run()
    out, lse = dc.results()
    ref_fn = lambda rr: O.chunk_prefill(case.q, kp, vp, case.block_table, case.cu_seqlens_q,  # noqa: E731
                                        case.kv_lens, case.scale, dtype="bf16", rows=rr,
                                        kr_pool=pools[2] if len(pools) == 3 else None)
    if rows is None:
        ref, ref_lse = OR.all_rows(ref_fn, case.T, block=128)
    else:
        ref, ref_lse = ref_fn(rows)
        out, lse = out[rows], lse[rows]
    e_out = gu.max_abs_err(out, ref)
    e_lse = gu.lse_err(lse, ref_lse)
    gu.announce(f"  max-abs-err out {e_out:.3e} lse {e_lse:.3e} (tol {tol:g}, lse {LSE_TOL:g}) "
                f"rows={'all' if rows is None else len(rows)}")
    assert e_out <= tol and e_lse <= LSE_TOL, (e_out, e_lse)
    return dc, out, lse


def test_chunk_config_full_size(gu):
    """Every row and head of the chunked-prefill workload (8 x 512-token chunks
    over 1024..6144-token cached prefixes, 32 query heads)."""
    _run(gu, gen.prefill_chunk_bf16())


def test_mla_chunk_config_full_size(gu):
    """Every row and head of the MLA chunked-prefill workload (rope keys from
    the paged rope cache)."""
    _run(gu, gen.prefill_chunk_mla_bf16())


@pytest.mark.parametrize("Hq,Hk", [(8, 8), (8, 2), (16, 1)])
def test_chunk_small_ragged(gu, Hq, Hk):
    """Prefixes that start and end inside pages, chunks shorter and longer than
    a 128-row query tile, a chunk that fills its sequence (no prefix)."""
    case = gen.make_chunk_case(name="chunk_small", seed=61, prefix_lens=[0, 1, 63, 64, 100, 255, 700],
                               q_lens=[5, 64, 1, 130, 129, 200, 300], Hq=Hq, Hk=Hk)
    _run(gu, case)


@pytest.mark.parametrize("seed", [71, 72, 73])
def test_chunk_grids_ranked_by_key_count(gu, seed):
    """Grids of more than two workgroups per compute unit (64 heads) rank
    their items by the keys each query tile sees.  Seeded random batches:
    prefixes 0..3000 (inside and across pages), chunks 0..400 tokens (some
    empty, some one token), every row and head compared."""
    rng = np.random.default_rng(seed)
    B = int(rng.integers(6, 12))
    prefix = [int(x) for x in rng.integers(0, 3001, size=B)]
    q_lens = [int(x) for x in rng.integers(0, 401, size=B)]
    q_lens[0], q_lens[1] = 0, 1
    q_lens[2] = max(q_lens[2], 260)  # at least one sequence with three query tiles
    case = gen.make_chunk_case(name=f"chunk_ranked_{seed}", seed=seed, prefix_lens=prefix, q_lens=q_lens,
                               Hq=64, Hk=8)
    items = sum(-(-q // 128) for q in q_lens)
    assert 64 * items > 512, "the grid must run in more than one round"
    _run(gu, case)


def test_chunk_empty_chunks_and_one_token_chunks(gu):
    case = gen.make_chunk_case(name="chunk_edges", seed=62, prefix_lens=[10, 0, 500, 64, 3],
                               q_lens=[0, 1, 1, 0, 257], Hq=8, Hk=2)
    _run(gu, case)


def test_one_token_chunks_equal_decode(gu):
    """q_len = 1 for every sequence: the chunk result is the decode result."""
    case = gen.make_chunk_case(name="chunk_decode", seed=63, prefix_lens=[1023, 64, 5, 300],
                               q_lens=[1, 1, 1, 1], Hq=16, Hk=4)
    dc, out, lse = _run(gu, case)
    kp, vp = dc.pools_bits()[:2]
    ref, ref_lse = O.paged_decode(case.q, kp, vp, case.block_table, case.kv_lens, case.scale, q_dtype="bf16",
                                  kv_dtype="bf16")
    assert gu.max_abs_err(out, ref) <= TOL and gu.lse_err(lse, ref_lse) <= LSE_TOL


def test_two_chunks_equal_one_prefill(gu):
    """One sequence prefilled in two chunks through the cache (append, attend,
    append, attend) gives the oracle's one-shot causal prefill of the whole
    sequence."""
    L, c = 700, 300
    full = gen.make_prefill_case(name="chunk_split_ref", seed=64, seq_lens=[L], Hq=8, Hk=2, D_qk=128, D_rope=0,
                                 D_v=128)
    ref_out, ref_lse = O.ragged_prefill(full.q, full.k, full.v, full.cu_seqlens, full.scale, dtype="bf16")
    # the same tokens as a paged cache, appended in two chunks
    case = gen.make_chunk_case(name="chunk_split", seed=65, prefix_lens=[0], q_lens=[c], Hq=8, Hk=2)
    pieces = []
    cache_k, cache_v = None, None
    for lo, hi in ((0, c), (c, L)):
        case.q = full.q[lo:hi]
        case.k_new = full.k[lo:hi]
        case.v_new = full.v[lo:hi]
        case.cu_seqlens_q = np.array([0, hi - lo], np.int32)
        case.kv_lens = np.array([hi], np.int32)
        nblk = (L + 63) // 64
        if cache_k is None:
            case.block_table = np.array([np.random.default_rng(66).permutation(nblk + 3)[:nblk]], np.int32)
            cache_k = np.full((nblk + 3, 2, 64, 128), 0x7FC0, np.uint16)
            cache_v = cache_k.copy()
        case.k_pool, case.v_pool = cache_k, cache_v
        gu.announce(f"chunk split rows {lo}..{hi}")
        dc = gu.DeviceChunk(case)
        dc.append()
        dc.run()
        pieces.append(dc.results())
        cache_k, cache_v = dc.pools_bits()
    out = np.concatenate([p[0] for p in pieces])
    lse = np.concatenate([p[1] for p in pieces])
    e_out, e_lse = gu.max_abs_err(out, ref_out), gu.lse_err(lse, ref_lse)
    gu.announce(f"  two chunks vs one prefill: out {e_out:.3e} lse {e_lse:.3e}")
    assert e_out <= TOL and e_lse <= LSE_TOL


def test_chunk_long_prefix_sampled(gu):
    """A 9000-key cache (more than 128 pages: two block-table words) and a
    600-token chunk."""
    case = gen.make_chunk_case(name="chunk_long", seed=67, prefix_lens=[8400, 40], q_lens=[600, 40], Hq=8, Hk=1)
    _run(gu, case, rows=_rows_sample(case))


@pytest.mark.parametrize("Hq,Hk", [(16, 16), (8, 2)])
def test_mla_chunk_rope_from_cache(gu, Hq, Hk):
    """MLA: Q 192 = 128 + 64 rope, the rope keys appended to and read from a
    one-head rope cache on the same pages."""
    case = gen.make_chunk_case(name="chunk_mla", seed=68, prefix_lens=[0, 63, 130, 700], q_lens=[5, 129, 64, 300],
                               Hq=Hq, Hk=Hk, D_rope=64)
    _run(gu, case)


def test_mla_chunk_long_prefix_sampled(gu):
    case = gen.make_chunk_case(name="chunk_mla_long", seed=69, prefix_lens=[5000, 1], q_lens=[512, 127], Hq=16,
                               Hk=16, D_rope=64)
    _run(gu, case, rows=_rows_sample(case))
