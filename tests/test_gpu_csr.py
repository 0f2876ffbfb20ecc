"""CSR page input on the GPU: gqap_block_table_from_csr builds the padded
block table from (kv_indices, kv_page_indptr) bit for bit like the oracle, and
decode and chunked prefill driven through it match the padded-table runs
exactly (same kernels, same pool block ids)."""
import numpy as np
import pytest
import torch

from oracle import attention as O
from workloads import gen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from tests import gpu_util  # imports the HIP library; fails loudly if it is missing
    return gpu_util


def _csr_of(table, lens):
    counts = [(int(L) + 63) // 64 for L in lens]
    idx = np.concatenate([table[b, :c] for b, c in enumerate(counts)] + [np.zeros(0, np.int32)]).astype(np.int32)
    indptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return idx, indptr


def _device_table(gu, idx, indptr, B, width, stride):
    gi = torch.from_numpy(idx if idx.size else np.zeros(1, np.int32)).cuda()
    gp = torch.from_numpy(indptr).cuda()
    out = torch.full((B, stride), 12345, dtype=torch.int32, device="cuda")
    gu.gq.gqap_block_table_from_csr(gi, gp, B, width, out, block_table_stride=stride)
    torch.cuda.synchronize()
    return out


def test_csr_table_matches_oracle_bit_exactly(gu):
    rng = np.random.default_rng(90)
    lens = [0, 1, 64, 65, 4000, 130]
    width = 70
    table = rng.permutation(500)[: len(lens) * width].reshape(len(lens), width).astype(np.int32)
    idx, indptr = _csr_of(table, lens)
    gu.announce(f"csr table lens={lens} pages={idx.size}")
    got = _device_table(gu, idx, indptr, len(lens), width, width + 3).cpu().numpy()
    ref = O.block_table_from_csr(idx, indptr, width)
    np.testing.assert_array_equal(got[:, :width], ref)
    assert np.all(got[:, width:] == 12345), "the row padding past the width was written"


def test_decode_through_csr_equals_padded_table(gu):
    case = gen.make_decode_case(name="csr_decode", seed=91, B=6, Hq=16, Hk=4, D=128, q_dtype="bf16",
                                kv_dtype="bf16", seq_lens=[5, 64, 700, 1, 129, 2048])
    gu.announce("csr decode")
    dd = gu.DeviceDecode(case)
    dd.run()
    ref_out, ref_lse = dd.results()
    idx, indptr = _csr_of(case.block_table, case.seq_lens)
    dd.bt = _device_table(gu, idx, indptr, case.B, case.block_table.shape[1], case.block_table.shape[1])
    dd.out.zero_()
    dd.run()
    out, lse = dd.results()
    np.testing.assert_array_equal(out, ref_out)
    np.testing.assert_array_equal(lse, ref_lse)


def test_chunk_prefill_through_csr_equals_padded_table(gu):
    case = gen.make_chunk_case(name="csr_chunk", seed=92, prefix_lens=[100, 0, 640], q_lens=[28, 64, 129], Hq=8,
                               Hk=2)
    gu.announce("csr chunked prefill")
    dc = gu.DeviceChunk(case)
    dc.append()
    dc.run()
    ref_out, ref_lse = dc.results()
    idx, indptr = _csr_of(case.block_table, case.kv_lens)
    dc.bt = _device_table(gu, idx, indptr, case.B, case.block_table.shape[1], case.block_table.shape[1])
    dc.out.zero_()
    dc.run()
    out, lse = dc.results()
    np.testing.assert_array_equal(out, ref_out)
    np.testing.assert_array_equal(lse, ref_lse)
