"""Paged decode on the GPU through the C ABI, against the fp64 oracle.

Tolerances (max-abs-err of out and lse against the oracle run on the same
rounded inputs): 1e-5 for fp32 inputs, 2e-2 for bf16, 6e-2 for fp8 KV."""
import numpy as np
import pytest
import torch

from oracle import attention as O
from oracle import parallel as OR
from workloads import gen

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2, "e4m3fn": 6e-2}
# The LSE is fp32 from end to end: 1e-3 catches a dropped or repeated block.
LSE_TOL = {"f32": 1e-5, "bf16": 1e-3, "e4m3fn": 1e-3}


@pytest.fixture(scope="module")
def gu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from tests import gpu_util  # imports the HIP library; fails loudly if it is missing
    return gpu_util


def _oracle(case, batches=None):
    if batches is None and case.B > 16:
        return OR.all_batches(lambda bb: _oracle(case, bb), case.B)
    return O.paged_decode(case.q, case.k_pool, case.v_pool, case.block_table, case.seq_lens, case.scale,
                          q_dtype=case.q_dtype, kv_dtype=case.kv_dtype, k_scale=case.k_scale,
                          v_scale=case.v_scale, batches=batches)


def _check(gu, case, num_workers=0, batches=None, tol=None):
    gu.announce(f"decode {case.name} B={case.B} Hq={case.Hq} Hk={case.Hk} D={case.D} kv={case.kv_dtype} "
                f"workers={num_workers} seed={case.meta.get('seed')}")
    dd = gu.DeviceDecode(case, num_workers=num_workers)
    dd.run()
    out, lse = dd.results()
    ref_out, ref_lse = _oracle(case, batches)
    if batches is not None:
        out, lse = out[batches], lse[batches]
    tol = TOL[case.kv_dtype] if tol is None else tol
    e_out = gu.max_abs_err(out, ref_out)
    e_lse = gu.lse_err(lse, ref_lse)
    gu.announce(f"  max-abs-err out {e_out:.3e} lse {e_lse:.3e} (tol {tol:g}) workers={dd.plan.num_workers}")
    assert e_out <= tol and e_lse <= min(tol, LSE_TOL[case.kv_dtype]), (e_out, e_lse)
    return dd, out, lse


def test_decode_tiny_fp32_config(gu):
    _check(gu, gen.decode_tiny_fp32())


def test_decode_gqa_bf16_config_full_size(gu):
    _check(gu, gen.decode_gqa_bf16())


def test_decode_long_fp8_config_full_size(gu):
    """All 128 sequences and 64 heads of the long fp8 workload."""
    _check(gu, gen.decode_long_fp8())


@pytest.mark.parametrize("kv", ["f32", "bf16", "e4m3fn"])
@pytest.mark.parametrize("D", [64, 128])
def test_decode_ragged_lengths(gu, kv, D):
    q_dtype = "f32" if kv == "f32" else "bf16"
    case = gen.make_decode_case(name=f"ragged_{kv}_{D}", seed=40 + D, B=7, Hq=32, Hk=8, D=D, q_dtype=q_dtype,
                                kv_dtype=kv, seq_lens=[1, 63, 64, 65, 200, 333, 1000])
    _check(gu, case)


@pytest.mark.parametrize("Hq,Hk", [(8, 8), (16, 1), (64, 2), (40, 8)])
def test_decode_head_ratios(gu, Hq, Hk):
    case = gen.make_decode_case(name=f"ratio_{Hq}_{Hk}", seed=50 + Hq, B=3, Hq=Hq, Hk=Hk, D=128, q_dtype="bf16",
                                kv_dtype="bf16", seq_lens=[17, 130, 777])
    _check(gu, case)


def test_decode_worker_count_invariance_fp32(gu):
    case = gen.make_decode_case(name="splits_f32", seed=61, B=4, Hq=8, Hk=2, D=128, q_dtype="f32",
                                kv_dtype="f32", seq_lens=[64 * 9 + 5, 1, 300, 64 * 12])
    outs = []
    for nw in (1, 2, 5, 12, 77, 0):
        _, out, lse = _check(gu, case, num_workers=nw)
        outs.append((out, lse))
    for out, lse in outs[1:]:
        assert np.abs(out - outs[0][0]).max() <= 1e-6
        assert np.abs(lse - outs[0][1]).max() <= 1e-6


@pytest.mark.parametrize("kv", ["bf16", "e4m3fn"])
def test_decode_worker_count_invariance_mfma(gu, kv):
    case = gen.make_decode_case(name=f"splits_{kv}", seed=62, B=4, Hq=16, Hk=2, D=128, q_dtype="bf16",
                                kv_dtype=kv, seq_lens=[64 * 20 + 5, 3, 900, 64 * 32])
    for nw in (1, 3, 8, 32, 131, 1000, 0):
        _check(gu, case, num_workers=nw)


@pytest.mark.parametrize("kv", ["f32", "bf16", "e4m3fn"])
def test_decode_block_shuffle_is_bit_identical(gu, kv):
    q_dtype = "f32" if kv == "f32" else "bf16"
    case = gen.make_decode_case(name=f"shuffle_{kv}", seed=70, B=5, Hq=16, Hk=4, D=128, q_dtype=q_dtype,
                                kv_dtype=kv, seq_lens=[5, 64, 129, 700, 1500])
    gu.announce(f"block shuffle {kv}")
    a = gu.DeviceDecode(case)
    a.run()
    out1, lse1 = a.results()
    perm = np.random.default_rng(1).permutation(case.NB)
    kp = np.empty_like(case.k_pool)
    vp = np.empty_like(case.v_pool)
    kp[perm] = case.k_pool
    vp[perm] = case.v_pool
    bt = np.where(case.block_table >= 0, perm[np.maximum(case.block_table, 0)], -1).astype(np.int32)
    case2 = gen.DecodeCase(**{**case.__dict__, "k_pool": kp, "v_pool": vp, "block_table": bt})
    b = gu.DeviceDecode(case2)
    b.run()
    out2, lse2 = b.results()
    assert np.array_equal(out1, out2) and np.array_equal(lse1, lse2)


@pytest.mark.parametrize("kv", ["f32", "bf16"])
def test_decode_seq_len_one_returns_the_value_row_exactly(gu, kv):
    q_dtype = "f32" if kv == "f32" else "bf16"
    case = gen.make_decode_case(name=f"len1_{kv}", seed=80, B=4, Hq=8, Hk=4, D=128, q_dtype=q_dtype,
                                kv_dtype=kv, seq_lens=[1, 1, 1, 1])
    gu.announce(f"seq_len=1 {kv}")
    dd = gu.DeviceDecode(case)
    dd.run()
    out, lse = dd.results()
    for b in range(case.B):
        for h in range(case.Hq):
            row = O.widen(case.v_pool[case.block_table[b, 0], h // 2, 0], kv)
            assert np.array_equal(out[b, h], row), (b, h)


def test_decode_head_mapping_8_to_4(gu):
    case = gen.make_decode_case(name="headmap", seed=90, B=2, Hq=8, Hk=4, D=128, q_dtype="bf16",
                                kv_dtype="bf16", seq_lens=[100, 37])
    vp = case.v_pool.copy()
    for g in range(4):                       # V of kv head g is the constant g + 1 (exact in bf16)
        vp[:, g] = np.float32(g + 1).view(np.uint32) >> 16
    case = gen.DecodeCase(**{**case.__dict__, "v_pool": vp})
    gu.announce("head mapping 8:4")
    dd = gu.DeviceDecode(case)
    dd.run()
    out, _ = dd.results()
    for h in range(8):
        assert np.abs(out[:, h] - (h // 2 + 1)).max() <= 1e-2, h


def test_decode_zero_length_sequence(gu):
    case = gen.make_decode_case(name="zero_len", seed=91, B=3, Hq=8, Hk=2, D=128, q_dtype="bf16",
                                kv_dtype="bf16", seq_lens=[0, 70, 0])
    dd, out, lse = _check(gu, case)
    assert np.all(out[0] == 0) and np.all(out[2] == 0)
    assert np.all(np.isneginf(lse[0])) and np.all(np.isneginf(lse[2]))


def test_decode_full_table_maximum_length(gu):
    case = gen.make_decode_case(name="full_table", seed=92, B=2, Hq=16, Hk=2, D=128, q_dtype="bf16",
                                kv_dtype="e4m3fn", seq_lens=[64 * 40, 64 * 40], nblk=40)
    _check(gu, case)


@pytest.mark.parametrize("kv", ["f32", "bf16", "e4m3fn"])
def test_debug_gather_matches_oracle_gather_bit_exactly(gu, kv):
    q_dtype = "f32" if kv == "f32" else "bf16"
    case = gen.make_decode_case(name=f"gather_{kv}", seed=93, B=3, Hq=8, Hk=4, D=128, q_dtype=q_dtype,
                                kv_dtype=kv, seq_lens=[1, 191, 640])
    gu.announce(f"debug gather {kv}")
    dd = gu.DeviceDecode(case)
    for b in range(case.B):
        L = int(case.seq_lens[b])
        for g in range(case.Hk):
            for pool, name in ((dd.k, "k"), (dd.v, "v")):
                dst = torch.zeros((max(L, 1), case.D), dtype=pool.dtype, device="cuda")
                import gqa_attention_paged_amd as gq
                gq.gqap_debug_gather_kv(dd.plan, pool, dd.bt, dd.sl, b, g, L, dst)
                torch.cuda.synchronize()
                got = dst[:L].cpu().view(torch.uint8).numpy().tobytes()
                src = case.k_pool if name == "k" else case.v_pool
                ref = np.ascontiguousarray(O.gather_kv_rows(src, case.block_table, b, g, L)).tobytes()
                assert got == ref, (b, g, name)


def test_decode_runs_on_a_side_stream(gu):
    case = gen.make_decode_case(name="stream", seed=94, B=2, Hq=8, Hk=2, D=128, q_dtype="bf16",
                                kv_dtype="bf16", seq_lens=[300, 45])
    gu.announce("side stream")
    dd = gu.DeviceDecode(case)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        dd.run(stream=s)
    s.synchronize()
    out, lse = dd.results()
    ref_out, ref_lse = _oracle(case)
    assert gu.max_abs_err(out, ref_out) <= TOL["bf16"]


def test_decode_very_long_sequence(gu):
    """One 131072-token sequence (2048 pages: block-table reads far past the
    first words, long prefix sums, many pieces per head) next to a 3-token one."""
    case = gen.make_decode_case(name="very_long", seed=95, B=2, Hq=8, Hk=1, D=128, q_dtype="bf16",
                                kv_dtype="bf16", seq_lens=[131072, 3])
    _check(gu, case)


@pytest.mark.parametrize("kv", ["bf16", "e4m3fn"])
def test_decode_many_short_sequences(gu, kv):
    """1000 sequences of 0..200 tokens: far more sequences than a wave has lanes,
    many of them inside one page, some empty."""
    rng = np.random.default_rng(96)
    lens = rng.integers(0, 201, size=1000)
    lens[::97] = 0
    case = gen.make_decode_case(name=f"many_{kv}", seed=96, B=1000, Hq=16, Hk=4, D=128, q_dtype="bf16",
                                kv_dtype=kv, seq_lens=lens.tolist())
    _check(gu, case)
