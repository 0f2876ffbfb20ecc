"""The C ABI at its edges, on the GPU: inputs past the plan's capacity, and
tensors with padded (non-contiguous) strides.

Capacity (include/gqap.h): a decode sequence whose length lies outside
[0, max_seq_len] is treated as empty (out 0, lse -inf); prefill rows past
max_seq_len, chunk rows past max_q_len, and every row of a chunk whose keys
exceed max_kv_len (or that is longer than its keys) get out 0 and lse -inf,
and such a chunk is not appended.  Output buffers start as NaN, so a row the
library leaves unwritten fails the test.

Strides: FlashMLA "Memory Layout Requirements" lets the batch, head and
sequence dimensions be strided as long as the last dimension is contiguous;
every descriptor takes element strides.  The strided runs read NaN-filled
padding around every row they do not own, so an address mix-up shows up as
NaN, and the padding of the outputs must still be NaN afterwards."""
import numpy as np
import pytest
import torch

from oracle import attention as O
from workloads import gen

pytestmark = pytest.mark.gpu

TOL = 2e-2
LSE_TOL = 1e-3
NAN = float("nan")


@pytest.fixture(scope="module")
def gu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from tests import gpu_util  # imports the HIP library; fails loudly if it is missing
    return gpu_util


@pytest.fixture(scope="module")
def gq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import gqa_attention_paged_amd
    return gqa_attention_paged_amd


def _padded(t: torch.Tensor, pad_mid: int = 1, pad_last: int = 64) -> torch.Tensor:
    """A view with t's values inside a NaN buffer: the second dimension has
    pad_mid extra (unowned) entries and the last pad_last extra columns, so
    every outer stride is larger than the packed one."""
    shape = list(t.shape)
    base_shape = shape[:1] + [shape[1] + pad_mid] + shape[2:-1] + [shape[-1] + pad_last]
    base = torch.full(base_shape, NAN, dtype=t.dtype, device=t.device)
    view = base[(slice(None), slice(0, shape[1])) + (slice(None),) * (len(shape) - 3) + (slice(0, shape[-1]),)]
    view.copy_(t)
    return view


def _padded_pool(t: torch.Tensor, pad_heads: int = 1, pad_slab: int = 64) -> torch.Tensor:
    """A [NB, H, 64, D] pool whose (block, head) slabs stay contiguous 64 x D
    tiles, with pad_heads unowned slabs per block and pad_slab elements of
    padding after every slab."""
    NB, H, R, D = t.shape
    base = torch.full((NB, H + pad_heads, R * D + pad_slab), NAN, dtype=t.dtype, device=t.device)
    view = base[:, :H, :R * D].view(NB, H, R, D)
    view.copy_(t)
    return view


def _padding_untouched(view: torch.Tensor) -> bool:
    """Every element of the view's buffer outside the view is still NaN."""
    base = torch.as_strided(view, (view.untyped_storage().nbytes() // view.element_size(),), (1,), 0)
    mask = torch.ones_like(base, dtype=torch.bool)
    idx = torch.as_strided(torch.arange(base.numel(), device=view.device), view.shape, view.stride(),
                           view.storage_offset())
    mask[idx.flatten()] = False
    return bool(torch.isnan(base[mask].float()).all())


# ---------------------------------------------------------------- capacity

def test_decode_lengths_outside_the_capacity_give_empty_rows(gu):
    """Plan capacity 200 keys; sequence 1 has 300 and sequence 3 a negative
    length: both come out as empty sequences; the others match the oracle."""
    case = gen.make_decode_case(name="decode_cap", seed=400, B=4, Hq=16, Hk=4, D=128, q_dtype="bf16",
                                kv_dtype="bf16", seq_lens=[100, 300, 37, 64])
    gu.announce("decode capacity: seq_lens [100, 300, 37, -5] against max_seq_len 200")
    dd = gu.DeviceDecode(case, max_seq_len=200)
    dd.sl[3] = -5
    dd.out.fill_(NAN)
    dd.lse.fill_(NAN)
    dd.run()
    out, lse = dd.results()
    for b in (1, 3):
        assert np.all(out[b] == 0) and np.all(np.isneginf(lse[b])), b
    keep = [0, 2]
    ref, ref_lse = O.paged_decode(case.q, case.k_pool, case.v_pool, case.block_table, case.seq_lens, case.scale,
                                  q_dtype="bf16", kv_dtype="bf16", batches=keep)
    assert gu.max_abs_err(out[keep], ref) <= TOL and gu.lse_err(lse[keep], ref_lse) <= LSE_TOL


@pytest.mark.parametrize("kind", ["plain", "head_pairs", "split"])
def test_prefill_rows_past_the_capacity_are_zero(gu, kind):
    """Plan capacity 256 rows: rows past it are 0 / -inf; the rows below it
    match the oracle (causality keeps them independent of the rows cut)."""
    mask = 0.5 if kind == "head_pairs" else None
    case = gen.make_prefill_case(name=f"prefill_cap_{kind}", seed=401, seq_lens=[300, 100, 500, 256], Hq=8,
                                 Hk=4 if kind == "head_pairs" else 2, D_qk=192 if kind == "split" else 128,
                                 D_rope=64 if kind == "split" else 0, D_v=128, mask_density=mask)
    gu.announce(f"prefill capacity {kind}: lens {case.seq_lens.tolist()} against max_seq_len 256")
    dp = gu.DevicePrefill(case, max_seq_len=256, num_splits=3 if kind == "split" else 0)
    assert dp.plan.q_tile_rows == (64 if kind == "head_pairs" else 128)
    dp.out.fill_(NAN)
    dp.lse.fill_(NAN)
    dp.run()
    out, lse = dp.results()
    cu = case.cu_seqlens
    rows_in = np.concatenate([np.arange(cu[b], cu[b] + min(256, case.seq_lens[b])) for b in range(case.B)])
    rows_cut = np.setdiff1d(np.arange(case.T), rows_in)
    assert rows_cut.size == 44 + 244
    assert np.all(out[rows_cut] == 0) and np.all(np.isneginf(lse[rows_cut]))
    ref, ref_lse = O.ragged_prefill(case.q, case.k, case.v, case.cu_seqlens, case.scale, k_rope=case.k_rope,
                                    block_mask=case.block_mask, dtype="bf16", rows=rows_in)
    e_out, e_lse = gu.max_abs_err(out[rows_in], ref), gu.lse_err(lse[rows_in], ref_lse)
    gu.announce(f"  rows below the capacity: out {e_out:.3e} lse {e_lse:.3e}")
    assert e_out <= TOL and e_lse <= LSE_TOL


@pytest.mark.parametrize("num_splits", [1, 2])
def test_chunk_rows_and_chunks_past_the_capacity(gu, num_splits):
    """Plan capacities max_q_len 100, max_kv_len 1000.  Chunk 0 (150 tokens)
    keeps its first 100 rows, computed with the causal offset of the whole
    chunk (kv_len - 150), and its last 50 rows are 0 / -inf; chunk 2 has 1300
    keys, past the capacity: all its rows are 0 / -inf and it is not
    appended; chunk 1 is ordinary."""
    case = gen.make_chunk_case(name="chunk_cap", seed=402, prefix_lens=[400, 64, 1200], q_lens=[150, 30, 100],
                               Hq=8, Hk=2)
    gu.announce(f"chunk capacity: kv_lens {case.kv_lens.tolist()} q_lens {case.q_lens.tolist()} splits={num_splits}")
    dc = gu.DeviceChunk(case, max_q_len=100, max_kv_len=1000, num_splits=num_splits, validate=False)
    dc.out.fill_(NAN)
    dc.lse.fill_(NAN)
    dc.append()
    kp, vp = dc.pools_bits()
    # the oracle's append of the two chunks inside the capacity only
    sub = gen.ChunkCase(**{**case.__dict__, "kv_lens": case.kv_lens[:2], "cu_seqlens_q": case.cu_seqlens_q[:3],
                           "block_table": case.block_table[:2]})
    want_k, want_v = O.append_kv(case.k_new, case.v_new, case.k_pool, case.v_pool, sub.block_table,
                                 sub.cu_seqlens_q, sub.kv_lens)
    assert np.array_equal(kp, want_k) and np.array_equal(vp, want_v), "append wrote outside the capacity"
    dc.run()
    out, lse = dc.results()
    cu = case.cu_seqlens_q
    cut = np.concatenate([np.arange(cu[0] + 100, cu[1]), np.arange(cu[2], cu[3])])
    assert np.all(out[cut] == 0) and np.all(np.isneginf(lse[cut]))
    keep = np.concatenate([np.arange(cu[0], cu[0] + 100), np.arange(cu[1], cu[2])])
    ref, ref_lse = O.chunk_prefill(case.q, want_k, want_v, case.block_table, case.cu_seqlens_q, case.kv_lens,
                                   case.scale, dtype="bf16", rows=keep)
    e_out, e_lse = gu.max_abs_err(out[keep], ref), gu.lse_err(lse[keep], ref_lse)
    gu.announce(f"  rows inside the capacity: out {e_out:.3e} lse {e_lse:.3e}")
    assert e_out <= TOL and e_lse <= LSE_TOL


def test_chunk_capacity_edges_in_a_grid_ranked_by_key_count(gu):
    """64 heads over 10 one-tile chunks: 640 workgroups, more than two per
    compute unit, so the kernel ranks its items by the keys they see.  The
    batch holds the edge cases of that ranking: a chunk longer than
    max_q_len 100 (its last 50 rows 0 / -inf), an empty chunk, a one-token
    chunk, a chunk with no cached prefix, a chunk exactly at the capacity,
    and last a chunk whose 1300 keys exceed max_kv_len 1000 (all rows 0 /
    -inf, not appended)."""
    prefix = [400, 64, 7, 300, 0, 900, 5, 333, 20, 1200]
    q_lens = [150, 30, 0, 1, 64, 99, 17, 77, 100, 100]
    case = gen.make_chunk_case(name="chunk_cap_ranked", seed=404, prefix_lens=prefix, q_lens=q_lens, Hq=64, Hk=8)
    gu.announce(f"chunk capacity, ranked grid: kv_lens {case.kv_lens.tolist()} q_lens {case.q_lens.tolist()}")
    dc = gu.DeviceChunk(case, max_q_len=100, max_kv_len=1000, validate=False)
    assert dc.plan.num_splits == 1
    dc.out.fill_(NAN)
    dc.lse.fill_(NAN)
    dc.append()
    kp, vp = dc.pools_bits()
    sub = gen.ChunkCase(**{**case.__dict__, "kv_lens": case.kv_lens[:9], "cu_seqlens_q": case.cu_seqlens_q[:10],
                           "block_table": case.block_table[:9]})
    want_k, want_v = O.append_kv(case.k_new, case.v_new, case.k_pool, case.v_pool, sub.block_table,
                                 sub.cu_seqlens_q, sub.kv_lens)
    assert np.array_equal(kp, want_k) and np.array_equal(vp, want_v), "append wrote outside the capacity"
    dc.run()
    out, lse = dc.results()
    cu = case.cu_seqlens_q
    cut = np.concatenate([np.arange(cu[0] + 100, cu[1]), np.arange(cu[9], cu[10])])
    assert np.all(out[cut] == 0) and np.all(np.isneginf(lse[cut]))
    keep = np.concatenate([np.arange(cu[0], cu[0] + 100), np.arange(cu[1], cu[9])])
    ref, ref_lse = O.chunk_prefill(case.q, want_k, want_v, case.block_table, case.cu_seqlens_q, case.kv_lens,
                                   case.scale, dtype="bf16", rows=keep)
    e_out, e_lse = gu.max_abs_err(out[keep], ref), gu.lse_err(lse[keep], ref_lse)
    gu.announce(f"  rows inside the capacity: out {e_out:.3e} lse {e_lse:.3e}")
    assert e_out <= TOL and e_lse <= LSE_TOL


# ---------------------------------------------------------------- strides

@pytest.mark.parametrize("kv", ["bf16", "e4m3fn"])
def test_decode_with_padded_strides(gu, gq, kv):
    case = gen.make_decode_case(name=f"decode_strided_{kv}", seed=410, B=5, Hq=16, Hk=4, D=128, q_dtype="bf16",
                                kv_dtype=kv, seq_lens=[1, 64, 200, 513, 1000])
    gu.announce(f"decode padded strides kv={kv}")
    dd = gu.DeviceDecode(case)
    dd.q = _padded(dd.q)
    dd.out = _padded(torch.empty_like(dd.out))
    if kv == "bf16":
        dd.k, dd.v = _padded_pool(dd.k), _padded_pool(dd.v)
    else:  # NaN code 0x7F in the padding of an fp8 pool
        kb, vb = dd.k.view(torch.uint8), dd.v.view(torch.uint8)
        for name, t in (("k", kb), ("v", vb)):
            NB, H, R, D = t.shape
            base = torch.full((NB, H + 1, R * D + 64), 0x7F, dtype=torch.uint8, device=t.device)
            view = base[:, :H, :R * D].view(NB, H, R, D)
            view.copy_(t)
            setattr(dd, name, view.view(torch.float8_e4m3fn))
    bt = torch.full((case.B, case.Nblk + 3), -1, dtype=torch.int32, device=dd.bt.device)
    bt[:, :case.Nblk] = dd.bt
    dd.bt = bt[:, :case.Nblk]
    assert dd.q.stride() != (case.Hq * 128, 128, 1) and dd.k.stride(1) > 64 * 128 and dd.bt.stride(0) > case.Nblk
    dd.desc = gq.decode_desc(dd.q, dd.k, dd.bt, max_seq_len=1000, out=dd.out)
    dd.plan = gq.gqap_decode_plan(dd.desc)
    dd.ws = torch.empty(dd.plan.workspace_bytes, dtype=torch.uint8, device=dd.q.device)
    dd.run()
    out, lse = dd.results()
    ref, ref_lse = O.paged_decode(case.q, case.k_pool, case.v_pool, case.block_table, case.seq_lens, case.scale,
                                  q_dtype="bf16", kv_dtype=kv, k_scale=case.k_scale, v_scale=case.v_scale)
    tol = TOL if kv == "bf16" else 6e-2
    assert gu.max_abs_err(out, ref) <= tol and gu.lse_err(lse, ref_lse) <= LSE_TOL
    assert _padding_untouched(dd.out)


@pytest.mark.parametrize("rope,mask", [(0, None), (64, None), (0, 0.4)])
def test_prefill_with_padded_strides(gu, gq, rope, mask):
    case = gen.make_prefill_case(name=f"prefill_strided_r{rope}", seed=411 + rope, seq_lens=[1, 130, 333, 64],
                                 Hq=8, Hk=8 if rope else 2, D_qk=128 + rope, D_rope=rope, D_v=128,
                                 mask_density=mask)
    gu.announce(f"prefill padded strides rope={rope} mask={mask}")
    dp = gu.DevicePrefill(case)
    dp.q, dp.k, dp.v = _padded(dp.q), _padded(dp.k, pad_mid=2), _padded(dp.v, pad_mid=1, pad_last=128)
    if rope:
        dp.kr = _padded(dp.kr, pad_mid=0, pad_last=64)
    dp.out = _padded(torch.empty_like(dp.out))
    dp.desc = gq.prefill_desc(dp.q, dp.k, dp.v, dp.kr, batch=case.B, max_seq_len=333, block_mask=dp.mask,
                              out=dp.out)
    dp.plan = gq.gqap_prefill_plan(dp.desc)
    dp.run()
    out, lse = dp.results()
    ref, ref_lse = O.ragged_prefill(case.q, case.k, case.v, case.cu_seqlens, case.scale, k_rope=case.k_rope,
                                    block_mask=case.block_mask, dtype="bf16")
    assert gu.max_abs_err(out, ref) <= TOL and gu.lse_err(lse, ref_lse) <= LSE_TOL
    assert _padding_untouched(dp.out)


@pytest.mark.parametrize("rope", [0, 64])
def test_chunk_with_padded_strides(gu, gq, rope):
    case = gen.make_chunk_case(name=f"chunk_strided_r{rope}", seed=413 + rope, prefix_lens=[0, 63, 300],
                               q_lens=[70, 129, 5], Hq=8, Hk=2 if rope == 0 else 8, D_rope=rope)
    gu.announce(f"chunk padded strides rope={rope}")
    dc = gu.DeviceChunk(case)
    dc.q = _padded(dc.q)
    dc.k_new, dc.v_new = _padded(dc.k_new, pad_mid=2), _padded(dc.v_new, pad_mid=2)
    dc.k_pool, dc.v_pool = _padded_pool(dc.k_pool), _padded_pool(dc.v_pool)
    if rope:
        dc.kr_new = _padded(dc.kr_new, pad_mid=0, pad_last=64)
        dc.kr_pool = _padded_pool(dc.kr_pool, pad_heads=0, pad_slab=256)
    dc.out = _padded(torch.empty_like(dc.out))
    dc.desc = gq.chunk_desc(dc.q, dc.k_new, dc.k_pool, dc.bt, batch=case.B, max_q_len=129,
                            max_kv_len=int(case.kv_lens.max()), out=dc.out, k_rope_new=dc.kr_new,
                            kr_pool=dc.kr_pool)
    assert dc.desc.kv_stride_head > 64 * 128 and dc.desc.new_stride_token > case.Hk * 128
    dc.plan = gq.gqap_chunk_plan(dc.desc)
    dc.append()
    pools = O.append_kv(case.k_new, case.v_new, case.k_pool, case.v_pool, case.block_table, case.cu_seqlens_q,
                        case.kv_lens, kr_new=case.kr_new, kr_pool=case.kr_pool)
    got = dc.pools_bits()
    assert all(np.array_equal(g, r) for g, r in zip(got, pools)), "strided append differs from the oracle's"
    assert _padding_untouched(dc.k_pool) and _padding_untouched(dc.v_pool)
    dc.run()
    out, lse = dc.results()
    ref, ref_lse = O.chunk_prefill(case.q, pools[0], pools[1], case.block_table, case.cu_seqlens_q, case.kv_lens,
                                   case.scale, dtype="bf16", kr_pool=pools[2] if rope else None)
    assert gu.max_abs_err(out, ref) <= TOL and gu.lse_err(lse, ref_lse) <= LSE_TOL
    assert _padding_untouched(dc.out)
