"""gqap_paged_decode_noalloc on the GPU, through the C ABI: the decode without
a caller workspace (its partial results live in the library's per-GPU scratch
array).  Two calls in a row, the second with a smaller input, each compared
with gqap_paged_decode on a caller workspace (the same kernels: bit-identical)
and with the oracle (2e-2 for bf16, 6e-2 for fp8 KV; LSE 1e-3).  Runs alone in
a fresh process or after the other tests."""
import numpy as np
import pytest
import torch

from oracle import attention as O
from oracle import parallel as OP
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


def _both(gu, case):
    gq = gu.gq
    dd = gu.DeviceDecode(case)
    assert dd.plan.workspace_bytes <= gq.NOALLOC_SCRATCH_BYTES
    dd.run()
    ref_out, ref_lse = dd.results()
    out = torch.full_like(dd.out, float("nan"))
    lse = torch.full_like(dd.lse, float("nan"))
    gq.gqap_paged_decode_noalloc(dd.plan, dd.q, dd.k, dd.v, dd.bt, dd.sl, case.scale, case.k_scale, case.v_scale,
                                 out, lse)
    torch.cuda.synchronize()
    got_out, got_lse = gu.tensor_to_f64(out), lse.cpu().numpy().astype(np.float64)
    return ref_out, ref_lse, got_out, got_lse


def _oracle(case):
    return OP.all_batches(lambda bb: O.paged_decode(case.q, case.k_pool, case.v_pool, case.block_table,
                                                    case.seq_lens, case.scale, q_dtype=case.q_dtype,
                                                    kv_dtype=case.kv_dtype, k_scale=case.k_scale,
                                                    v_scale=case.v_scale, batches=bb), case.B)


def test_noalloc_decode_two_calls_second_smaller(gu):
    cases = [gen.decode_long_fp8(), gen.decode_gqa_bf16(),
             gen.make_decode_case(name="noalloc_small", seed=420, B=5, Hq=16, Hk=4, D=128, q_dtype="bf16",
                                  kv_dtype="bf16", seq_lens=[1, 64, 65, 700, 3])]
    for case in cases:   # each call smaller than the one before it
        gu.announce(f"noalloc decode {case.name} B={case.B} Hq={case.Hq} kv={case.kv_dtype}")
        ref_out, ref_lse, out, lse = _both(gu, case)
        assert np.array_equal(out, ref_out) and np.array_equal(lse, ref_lse), case.name
        o_out, o_lse = _oracle(case)
        e_out, e_lse = gu.max_abs_err(out, o_out), gu.lse_err(lse, o_lse)
        gu.announce(f"  bit-identical to the workspace call; oracle out {e_out:.3e} lse {e_lse:.3e}")
        assert e_out <= TOL[case.kv_dtype] and e_lse <= LSE_TOL


def test_noalloc_decode_rejects_a_plan_past_the_scratch(gu):
    gq = gu.gq
    case = gen.make_decode_case(name="noalloc_big", seed=421, B=4, Hq=16, Hk=4, D=128, q_dtype="bf16",
                                kv_dtype="bf16", seq_lens=[64, 64, 64, 64])
    dd = gu.DeviceDecode(case, num_workers=20000)      # 20000+ pieces of 4 x 128 floats: past 32 MiB
    assert dd.plan.workspace_bytes > gq.NOALLOC_SCRATCH_BYTES
    with pytest.raises(gq.GqapError) as ei:
        gq.gqap_paged_decode_noalloc(dd.plan, dd.q, dd.k, dd.v, dd.bt, dd.sl, case.scale, 1.0, 1.0, dd.out, dd.lse)
    assert ei.value.status == gq.GQAP_ERR_UNSUPPORTED and "workspace" in str(ei.value)
