"""Seeded random shapes for every path, on the GPU through the C ABI, each
compared in full (every row and head) against the fp64 oracle.

The fixed cases of the other GPU tests pick their edges by hand; these draw
the sizes: batch, head counts and ratios (including ratios that are not
powers of two), head widths, dtypes, ragged lengths (0, 1, page edges and up
to a few thousand keys), worker counts, split counts, mask densities and
chunk lengths, so that the grids, tails and schedules meet combinations no
one chose.  The draws depend on the seed alone.  Bars as everywhere: fp32
1e-5, bf16 2e-2, fp8 6e-2 for the output; the fp32 LSE 1e-3 (fp32 decode
1e-5; fp8 Q.K prefill 1e-3 plus the summation bound of its scores)."""
import numpy as np
import pytest
import torch

from oracle import attention as O
from oracle import parallel as OR
from workloads import gen

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2, "e4m3fn": 6e-2}
LSE_TOL = 1e-3
EDGES = [0, 1, 2, 63, 64, 65, 127, 128, 129, 191, 255, 256, 257]


@pytest.fixture(scope="module")
def gu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from tests import gpu_util  # imports the HIP library; fails loudly if it is missing
    return gpu_util


def _lengths(rng, B, hi, allow_zero=True):
    out = []
    for _ in range(B):
        if rng.random() < 0.4:
            L = int(rng.choice(EDGES))
        else:
            L = int(rng.integers(1, hi + 1))
        out.append(L if (allow_zero or L > 0) else 1)
    return out


@pytest.mark.parametrize("seed", range(12))
def test_random_decode(gu, seed):
    rng = np.random.default_rng(5000 + seed)
    kv = ["f32", "bf16", "e4m3fn"][seed % 3]
    D = int(rng.choice([64, 128]))
    Hk = int(rng.choice([1, 2, 4, 8]))
    ratio = int(rng.choice([1, 2, 3, 4, 5, 8, 16, 24]))
    B = int(rng.integers(1, 41))
    lens = _lengths(rng, B, 3000)
    if sum(lens) == 0:      # the pool needs at least one block
        lens[0] = 1
    workers = int(rng.choice([0, 0, 7, 100, 1024, 3000]))
    case = gen.make_decode_case(name=f"rand_decode_{seed}", seed=5000 + seed, B=B, Hq=Hk * ratio, Hk=Hk, D=D,
                                q_dtype="f32" if kv == "f32" else "bf16", kv_dtype=kv, seq_lens=lens)
    gu.announce(f"random decode seed={seed} kv={kv} D={D} Hq={Hk * ratio} Hk={Hk} B={B} workers={workers} "
                f"lens={lens[:8]}")
    dd = gu.DeviceDecode(case, num_workers=workers)
    dd.out.fill_(float("nan"))
    dd.run()
    out, lse = dd.results()
    ref, ref_lse = OR.all_batches(lambda bb: O.paged_decode(case.q, case.k_pool, case.v_pool, case.block_table,
                                                            case.seq_lens, case.scale, q_dtype=case.q_dtype,
                                                            kv_dtype=kv, k_scale=case.k_scale,
                                                            v_scale=case.v_scale, batches=bb), B)
    e_out, e_lse = gu.max_abs_err(out, ref), gu.lse_err(lse, ref_lse)
    gu.announce(f"  out {e_out:.3e} lse {e_lse:.3e}")
    assert e_out <= TOL[kv] and e_lse <= (1e-5 if kv == "f32" else LSE_TOL), (e_out, e_lse)


@pytest.mark.parametrize("seed", range(10))
def test_random_prefill(gu, seed):
    """bf16 plain and MLA, fp8 nope parts (per tensor or per row), the
    quantised rope key; with or without a block mask; splits forced or not."""
    rng = np.random.default_rng(6000 + seed)
    kind = ["bf16", "mla", "fp8", "fp8_row", "rope8"][seed % 5]
    mla = kind != "bf16"
    Hk = int(rng.choice([1, 2, 4])) if not mla else int(rng.choice([1, 2, 4, 8]))
    ratio = int(rng.choice([1, 2, 3, 4])) if kind != "rope8" else 1
    if kind in ("fp8", "fp8_row"):
        ratio = int(rng.choice([1, 2, 4]))
    B = int(rng.integers(1, 7))
    lens = _lengths(rng, B, 900)
    if sum(lens) == 0:
        lens[0] = 5
    mask = float(rng.choice([0.2, 0.6])) if rng.random() < 0.4 else None
    splits = int(rng.choice([0, 0, 1, 2, 3]))
    Hq = Hk * ratio
    name = f"rand_prefill_{kind}_{seed}"
    if kind == "bf16":
        case = gen.make_prefill_case(name=name, seed=6000 + seed, seq_lens=lens, Hq=Hq, Hk=Hk, D_qk=128, D_rope=0,
                                     D_v=128, mask_density=mask)
    elif kind == "mla":
        case = gen.make_prefill_case(name=name, seed=6000 + seed, seq_lens=lens, Hq=Hq, Hk=Hk, D_qk=192,
                                     D_rope=64, D_v=128, mask_density=mask)
    elif kind == "rope8":
        case = gen.make_prefill_rope_fp8_case(name=name, seed=6000 + seed, seq_lens=lens, Hq=Hq, Hk=Hk,
                                              mask_density=mask)
    else:
        case = gen.make_prefill_fp8_case(name=name, seed=6000 + seed, seq_lens=lens, Hq=Hq, Hk=Hk,
                                         D_rope=int(rng.choice([0, 64])), mask_density=mask,
                                         blockwise=kind == "fp8_row")
    gu.announce(f"random prefill seed={seed} kind={kind} Hq={Hq} Hk={Hk} lens={lens} mask={mask} splits={splits}")
    dp = gu.DevicePrefill(case, num_splits=splits)
    dp.out.fill_(float("nan"))
    dp.run()
    out, lse = dp.results()
    if kind in ("fp8", "fp8_row"):
        fn = lambda rr: O.ragged_prefill_fp8(case.q, case.q_rope, case.k, case.v, case.k_rope,  # noqa: E731
                                             case.cu_seqlens, case.scale, case.q_scale, case.k_scale,
                                             block_mask=case.block_mask, rows=rr)
        from tests.test_gpu_prefill_fp8 import fp8_lse_bound
        lse_bound = fp8_lse_bound(case)
    elif kind == "rope8":
        fn = lambda rr: O.ragged_prefill_rope_fp8(case.q, case.k, case.v, case.k_rope,  # noqa: E731
                                                  case.k_rope_scale, case.cu_seqlens, case.scale,
                                                  block_mask=case.block_mask, rows=rr)
        lse_bound = LSE_TOL
    else:
        fn = lambda rr: O.ragged_prefill(case.q, case.k, case.v, case.cu_seqlens, case.scale,  # noqa: E731
                                         k_rope=case.k_rope, block_mask=case.block_mask, dtype="bf16", rows=rr)
        lse_bound = LSE_TOL
    ref, ref_lse = OR.all_rows(fn, case.T)
    tol = TOL["bf16"] if kind in ("bf16", "mla") else TOL["e4m3fn"]
    e_out = gu.max_abs_err(out, ref)
    ok_lse = gu.lse_within(lse, ref_lse, lse_bound)
    gu.announce(f"  out {e_out:.3e} lse {gu.lse_err(lse, ref_lse):.3e}")
    assert e_out <= tol and ok_lse, (e_out, gu.lse_err(lse, ref_lse))


@pytest.mark.parametrize("seed", range(10))
def test_random_chunk(gu, seed):
    """Chunks long and short (short ones may run on the decode workers),
    plain and MLA, over a bf16 or an fp8 cache, splits forced or not; the
    append checked bit for bit first."""
    rng = np.random.default_rng(7000 + seed)
    rope = 64 if seed % 3 == 1 else 0
    kv = "e4m3fn" if seed % 4 == 3 else "bf16"
    Hk = int(rng.choice([1, 2, 4]))
    ratio = int(rng.choice([1, 2, 4, 8])) if not rope else int(rng.choice([1, 2]))
    B = int(rng.integers(1, 7))
    short = rng.random() < 0.5
    qmax = max(1, 16 // ratio) if short else 300
    q_lens = [int(rng.integers(0, qmax + 1)) for _ in range(B)]
    prefix = _lengths(rng, B, 2500)
    splits = int(rng.choice([0, 0, 0, 1, 2]))
    case = gen.make_chunk_case(name=f"rand_chunk_{seed}", seed=7000 + seed, prefix_lens=prefix, q_lens=q_lens,
                               Hq=Hk * ratio, Hk=Hk, D_rope=rope, kv_dtype=kv)
    dc = gu.DeviceChunk(case, num_splits=splits)
    gu.announce(f"random chunk seed={seed} Hq={Hk * ratio} Hk={Hk} rope={rope} kv={kv} prefix={prefix} "
                f"q_lens={q_lens} splits={splits} kernel={dc.plan.kernel}")
    dc.out.fill_(float("nan"))
    dc.append()
    fp8 = kv == "e4m3fn"
    pools = O.append_kv(case.k_new, case.v_new, case.k_pool, case.v_pool, case.block_table, case.cu_seqlens_q,
                        case.kv_lens, kr_new=case.kr_new, kr_pool=case.kr_pool, kv_dtype=kv,
                        k_scale=case.k_scale if fp8 else 1.0, v_scale=case.v_scale if fp8 else 1.0)
    got = dc.pools_bits()
    for g, r in zip(got, pools):
        if fp8 and g.dtype == np.uint8:   # a NaN input may give either NaN code
            nan_g, nan_r = (g & 0x7F) == 0x7F, (r & 0x7F) == 0x7F
            assert np.array_equal(nan_g, nan_r) and np.array_equal(g[~nan_r], r[~nan_r]), "appended pool differs"
        else:
            assert np.array_equal(g, r), "appended pool differs from the oracle's"
    dc.run()
    out, lse = dc.results()
    kw = dict(kv_dtype="e4m3fn", k_scale=case.k_scale, v_scale=case.v_scale) if fp8 else {}
    fn = lambda rr: O.chunk_prefill(case.q, pools[0], pools[1], case.block_table, case.cu_seqlens_q,  # noqa: E731
                                    case.kv_lens, case.scale, dtype="bf16", rows=rr,
                                    kr_pool=pools[2] if rope else None, **kw)
    if case.T == 0:
        return
    ref, ref_lse = OR.all_rows(fn, case.T, block=64)
    e_out, e_lse = gu.max_abs_err(out, ref), gu.lse_err(lse, ref_lse)
    gu.announce(f"  out {e_out:.3e} lse {e_lse:.3e}")
    assert e_out <= TOL[kv] and e_lse <= LSE_TOL, (e_out, e_lse)
