"""The C ABI on the host: the library loads, exports every function that
include/gqap.h declares, its structures have the layout the binding assumes,
and planning / host validation reject exactly the calls they document.
No device calls are made here."""
import ctypes
import os
import re
import shutil
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gqap.h")
GOLDEN = os.path.join(ROOT, "tests", "golden", "precall_checks.txt")


@pytest.fixture(scope="module")
def gq():
    import gqa_attention_paged_amd as m  # raises ImportError when the library is not built
    return m


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(gqap_[a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_header_declares_the_binding_functions(gq):
    decl = declared_functions()
    assert decl, "no functions parsed from the header"
    assert sorted(gq.C_FUNCTIONS) == decl


def test_library_exports_every_declared_symbol(gq):
    lib = ctypes.CDLL(gq.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    nm = shutil.which("nm")
    if nm:
        out = subprocess.run([nm, "-D", "--defined-only", gq.LIB_PATH], capture_output=True, text=True).stdout
        exported = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
        for name in declared_functions():
            assert name in exported, name


def test_version_string(gq):
    assert "gfx950" in gq.gqap_version()


LAYOUT_PROGRAM = r"""
#include <stddef.h>
#include <stdio.h>
#include "gqap.h"
#define F(T, f) printf(#T " " #f " %zu\n", offsetof(T, f));
int main(void) {
  printf("gqap_decode_desc_t sizeof %zu\n", sizeof(gqap_decode_desc_t));
  printf("gqap_decode_plan_t sizeof %zu\n", sizeof(gqap_decode_plan_t));
  printf("gqap_prefill_desc_t sizeof %zu\n", sizeof(gqap_prefill_desc_t));
  printf("gqap_prefill_plan_t sizeof %zu\n", sizeof(gqap_prefill_plan_t));
  printf("gqap_chunk_desc_t sizeof %zu\n", sizeof(gqap_chunk_desc_t));
  printf("gqap_chunk_plan_t sizeof %zu\n", sizeof(gqap_chunk_plan_t));
  %FIELDS%
  return 0;
}
"""


def test_struct_layout_matches_the_c_compiler(gq, tmp_path):
    cc = shutil.which("gcc") or shutil.which("cc")
    if not cc:
        pytest.skip("no C compiler")
    structs = {"gqap_decode_desc_t": gq.DecodeDesc, "gqap_decode_plan_t": gq.DecodePlan,
               "gqap_prefill_desc_t": gq.PrefillDesc, "gqap_prefill_plan_t": gq.PrefillPlan,
               "gqap_chunk_desc_t": gq.ChunkDesc, "gqap_chunk_plan_t": gq.ChunkPlan}
    fields = "\n  ".join(f"F({cn}, {f})" for cn, py in structs.items() for f, _ in py._fields_)
    src = tmp_path / "layout.c"
    src.write_text(LAYOUT_PROGRAM.replace("%FIELDS%", fields))
    exe = tmp_path / "layout"
    subprocess.run([cc, "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), str(src), "-o",
                    str(exe)], check=True)
    got = {}
    for ln in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.splitlines():
        t, f, v = ln.split()
        got[(t, f)] = int(v)
    for cn, py in structs.items():
        assert got[(cn, "sizeof")] == ctypes.sizeof(py), cn
        for f, _ in py._fields_:
            assert got[(cn, f)] == getattr(py, f).offset, (cn, f)


# ---------------------------------------------------------------- decode planning

def baseline_decode_desc(gq):
    """B=64, Hq=32, Hk=8, D=128, 64 blocks per sequence, capacity 4096, bf16,
    contiguous [B, Hq, D] q/out and [NB, Hk, 64, D] pools."""
    d = gq.DecodeDesc()
    d.batch, d.num_q_heads, d.num_kv_heads, d.head_dim = 64, 32, 8, 128
    d.block_size, d.max_blocks_per_seq, d.num_pool_blocks, d.max_seq_len = 64, 64, 4096, 4096
    d.q_dtype = d.kv_dtype = gq.BF16
    d.q_stride_head, d.q_stride_batch = 128, 32 * 128
    d.out_stride_head, d.out_stride_batch = 128, 32 * 128
    d.kv_stride_head, d.kv_stride_block = 64 * 128, 8 * 64 * 128
    d.block_table_stride = 64
    return d


def golden_cases():
    cases = []
    for ln in open(GOLDEN):
        ln = ln.split("#", 1)[0].strip()
        if not ln:
            continue
        lhs, want = [p.strip() for p in ln.split("->")]
        parts = lhs.split()
        cases.append((parts[0], dict(p.split("=") for p in parts[1:]), want))
    return cases


@pytest.mark.parametrize("name,overrides,want", golden_cases(), ids=[c[0] for c in golden_cases()])
def test_decode_plan_precall_checks(gq, name, overrides, want):
    d = baseline_decode_desc(gq)
    for k, v in overrides.items():
        setattr(d, k, getattr(gq, v) if v in ("F32", "BF16", "FP8_E4M3FN", "F16") else int(v))
    status = gq.lib().gqap_decode_plan(ctypes.byref(d), ctypes.byref(gq.DecodePlan()))
    assert gq.STATUS_NAMES[status] == want, (name, gq.gqap_last_error())
    if want != "OK":
        assert gq.gqap_last_error(), "an error status leaves a message"


def test_decode_plan_is_a_function_of_the_descriptor(gq):
    d = baseline_decode_desc(gq)
    p = gq.gqap_decode_plan(d)
    assert p.magic == gq.PLAN_MAGIC and p.ratio == 4
    assert p.num_workers == 256 * 3        # D=128 bf16: three persistent waves per compute unit
    assert p.head_chunks == 1
    assert p.max_pieces == 64 * 8 * 1 + p.num_workers
    # prefix (B+1 ints), lse (pieces x 4 floats: one per query head of a KV head), partial
    # outputs (pieces x 4 x D floats), 256-byte rounded
    r = lambda n: (n + 255) // 256 * 256
    assert p.workspace_bytes == r(4 * 65) + r(4 * 4 * p.max_pieces) + r(4 * 4 * 128 * p.max_pieces)
    d.num_workers = 77
    assert gq.gqap_decode_plan(d).num_workers == 77
    d.num_workers, d.num_cus = 0, 80
    assert gq.gqap_decode_plan(d).num_workers == 80 * 3
    d.q_dtype = d.kv_dtype = gq.F32
    d.num_cus = 0
    assert gq.gqap_decode_plan(d).num_workers == 256 * 2


@pytest.mark.parametrize("field,value,status", [
    ("head_dim", 96, "UNSUPPORTED"), ("q_dtype", 7, "DTYPE"), ("kv_dtype", 3, "UNSUPPORTED"),
    ("max_blocks_per_seq", 0, "INVALID_ARGUMENT"), ("num_workers", -1, "INVALID_ARGUMENT"),
    ("batch", 65536, "INVALID_ARGUMENT"), ("kv_stride_head", 64 * 100, "INVALID_ARGUMENT"),
])
def test_decode_plan_rejects(gq, field, value, status):
    d = baseline_decode_desc(gq)
    setattr(d, field, value)
    got = gq.lib().gqap_decode_plan(ctypes.byref(d), ctypes.byref(gq.DecodePlan()))
    assert gq.STATUS_NAMES[got] == status, gq.gqap_last_error()


def test_decode_plan_accepts_an_empty_batch(gq):
    d = baseline_decode_desc(gq)
    d.batch = 0
    assert gq.gqap_decode_plan(d).magic == gq.PLAN_MAGIC


def test_validate_host_metadata(gq):
    d = baseline_decode_desc(gq)
    d.batch, d.num_pool_blocks = 2, 10
    p = gq.gqap_decode_plan(d)
    bt = np.full((2, 64), -1, np.int32)
    bt[0, :3] = [4, 9, 0]
    bt[1, :1] = [7]
    gq.gqap_decode_validate_host(p, bt, np.array([130, 64], np.int32))      # 3 blocks and 1 block: fine
    with pytest.raises(gq.GqapError, match="block_table"):
        gq.gqap_decode_validate_host(p, bt, np.array([130, 65], np.int32))  # needs a second block: -1
    bt[0, 1] = 10
    with pytest.raises(gq.GqapError, match="outside the pool"):
        gq.gqap_decode_validate_host(p, bt, np.array([130, 64], np.int32))
    bt[0, 1] = 9
    with pytest.raises(gq.GqapError, match="seq_lens"):
        gq.gqap_decode_validate_host(p, bt, np.array([4097, 0], np.int32))
    with pytest.raises(gq.GqapError, match="seq_lens"):
        gq.gqap_decode_validate_host(p, bt, np.array([-1, 0], np.int32))


def test_calls_reject_a_plan_that_was_never_made(gq):
    bad = gq.DecodePlan()
    st = gq.lib().gqap_paged_decode(ctypes.byref(bad), None, None, None, None, None, 1.0, 1.0, 1.0, None, None,
                                    None, 0, None)
    assert gq.STATUS_NAMES[st] == "INVALID_ARGUMENT"
    st = gq.lib().gqap_prefill(ctypes.byref(gq.PrefillPlan()), None, None, None, None, None, None, 1.0, None, None,
                               None, 0, None)
    assert gq.STATUS_NAMES[st] == "INVALID_ARGUMENT"


# ---------------------------------------------------------------- prefill planning

def baseline_prefill_desc(gq, mla=True):
    d = gq.PrefillDesc()
    Dqk, Dr = (192, 64) if mla else (128, 0)
    d.batch, d.num_q_heads, d.num_kv_heads = 4, 16, 16 if mla else 8
    d.head_dim_qk, d.head_dim_rope, d.head_dim_v = Dqk, Dr, 128
    d.total_tokens, d.max_seq_len, d.dtype, d.causal = 6584, 3000, gq.BF16, 1
    d.q_stride_head, d.q_stride_token = Dqk, Dqk * d.num_q_heads
    d.k_stride_head, d.k_stride_token = Dqk - Dr, (Dqk - Dr) * d.num_kv_heads
    d.v_stride_head, d.v_stride_token = 128, 128 * d.num_kv_heads
    d.kr_stride_token = Dr if Dr else 0
    d.out_stride_head, d.out_stride_token = 128, 128 * d.num_q_heads
    return d


def test_prefill_plan_baseline(gq):
    p = gq.gqap_prefill_plan(baseline_prefill_desc(gq))
    assert p.magic == gq.PLAN_MAGIC and p.q_tile_rows == 128 and p.q_tiles == 24 and p.workspace_bytes == 0
    d = baseline_prefill_desc(gq, mla=False)
    p = gq.gqap_prefill_plan(d)
    assert p.ratio == 2 and p.q_tile_rows == 128 and p.q_tiles == 24
    # with a block mask an even head ratio pairs the heads of a KV group: 64-row query tiles,
    # the same number of workgroups
    d.has_block_mask, d.mask_blocks = 1, 47
    p = gq.gqap_prefill_plan(d)
    assert p.q_tile_rows == 64 and p.q_tiles == 47
    d.num_kv_heads = 16                  # ratio 1: no pairs
    d.k_stride_token, d.v_stride_token = 128 * 16, 128 * 16
    p = gq.gqap_prefill_plan(d)
    assert p.q_tile_rows == 128 and p.q_tiles == 24


@pytest.mark.parametrize("field,value,status", [
    ("head_dim_rope", 0, "UNSUPPORTED"),        # 192 wide without the rope split
    ("head_dim_v", 64, "UNSUPPORTED"),
    ("dtype", 0, "DTYPE"),
    ("causal", 0, "UNSUPPORTED"),
    ("num_kv_heads", 3, "INVALID_ARGUMENT"),
    ("max_seq_len", 7000, "INVALID_ARGUMENT"),  # longer than the packed token count
    ("k_stride_token", 100, "INVALID_ARGUMENT"),
    ("q_stride_head", 200, "INVALID_ARGUMENT"),  # 16 heads of 200 overrun the 3072-element token stride
    ("has_block_mask", 2, "INVALID_ARGUMENT"),
    ("batch", -1, "INVALID_ARGUMENT"),
])
def test_prefill_plan_rejects(gq, field, value, status):
    d = baseline_prefill_desc(gq)
    setattr(d, field, value)
    got = gq.lib().gqap_prefill_plan(ctypes.byref(d), ctypes.byref(gq.PrefillPlan()))
    assert gq.STATUS_NAMES[got] == status, gq.gqap_last_error()


def test_prefill_plan_block_mask_extent(gq):
    d = baseline_prefill_desc(gq)
    d.has_block_mask, d.mask_blocks = 1, 46                  # ceil(3000 / 64) = 47 needed
    assert gq.lib().gqap_prefill_plan(ctypes.byref(d), ctypes.byref(gq.PrefillPlan())) != 0
    d.mask_blocks = 47
    assert gq.gqap_prefill_plan(d).magic == gq.PLAN_MAGIC


def baseline_fp8_prefill_desc(gq, mla=True):
    """The bf16 baseline with fp8 q_nope [T, 16, 128] and k codes, q_rope [T, 16, 64] bf16."""
    d = baseline_prefill_desc(gq, mla)
    d.dtype = gq.FP8_E4M3FN
    d.q_stride_head, d.q_stride_token = 128, 128 * d.num_q_heads
    if mla:
        d.qr_stride_head, d.qr_stride_token = 64, 64 * d.num_q_heads
    return d


def test_fp8_prefill_plan_baseline(gq):
    p = gq.gqap_prefill_plan(baseline_fp8_prefill_desc(gq))
    assert p.magic == gq.PLAN_MAGIC and p.kernel == 4 and p.q_tiles == 24
    assert gq.gqap_prefill_plan(baseline_fp8_prefill_desc(gq, mla=False)).kernel == 3


@pytest.mark.parametrize("field,value", [
    ("q_stride_head", 120),        # q_nope narrower than 128 codes
    ("q_stride_head", 136),        # 136-byte rows are not 16-byte aligned
    ("k_stride_token", 16 * 128 + 8),
    ("qr_stride_head", 32),        # q_rope narrower than the rope width
    ("qr_stride_token", 64 * 15),  # q_rope heads overlap
    ("qr_stride_head", 68),        # 136-byte bf16 rows
])
def test_fp8_prefill_plan_rejects(gq, field, value):
    d = baseline_fp8_prefill_desc(gq)
    setattr(d, field, value)
    got = gq.lib().gqap_prefill_plan(ctypes.byref(d), ctypes.byref(gq.PrefillPlan()))
    assert gq.STATUS_NAMES[got] == "INVALID_ARGUMENT", gq.gqap_last_error()


def test_prefill_entry_points_reject_the_other_dtype(gq):
    """gqap_prefill refuses an fp8 plan and gqap_prefill_fp8 a bf16 plan, before
    any device work (the pointers are never looked at)."""
    p8 = gq.gqap_prefill_plan(baseline_fp8_prefill_desc(gq))
    pb = gq.gqap_prefill_plan(baseline_prefill_desc(gq))
    st = gq.lib().gqap_prefill(ctypes.byref(p8), None, None, None, None, None, None, 1.0, None, None, None, 0, None)
    assert gq.STATUS_NAMES[st] == "DTYPE"
    st = gq.lib().gqap_prefill_fp8(ctypes.byref(pb), None, None, None, None, None, None, None, 1.0, 1.0, 1.0, None,
                                   None, None, 0, None)
    assert gq.STATUS_NAMES[st] == "DTYPE"


@pytest.mark.parametrize("scales", [(float("nan"), 1.0, 1.0), (1.0, float("inf"), 1.0), (1.0, 1.0, float("nan"))])
def test_fp8_prefill_rejects_non_finite_scales(gq, scales):
    p8 = gq.gqap_prefill_plan(baseline_fp8_prefill_desc(gq))
    st = gq.lib().gqap_prefill_fp8(ctypes.byref(p8), None, None, None, None, None, None, None, *scales, None, None,
                                   None, 0, None)
    assert gq.STATUS_NAMES[st] == "INVALID_ARGUMENT"


def test_fp8_blockwise_prefill_rejects(gq):
    p8 = gq.gqap_prefill_plan(baseline_fp8_prefill_desc(gq))
    pb = gq.gqap_prefill_plan(baseline_prefill_desc(gq))
    fake = 1 << 20  # never dereferenced: validation fails first
    call = gq.lib().gqap_prefill_fp8_blockwise
    st = call(ctypes.byref(pb), fake, fake, fake, fake, fake, fake, None, 1.0, fake, fake, fake, None, None, 0, None)
    assert gq.STATUS_NAMES[st] == "DTYPE"
    st = call(ctypes.byref(p8), fake, fake, fake, fake, fake, fake, None, 1.0, None, fake, fake, None, None, 0, None)
    assert gq.STATUS_NAMES[st] == "INVALID_ARGUMENT" and "scales" in gq.gqap_last_error()
    st = call(ctypes.byref(p8), fake, fake, fake, fake, fake, fake, None, 1.0, fake + 2, fake, fake, None, None, 0,
              None)
    assert gq.STATUS_NAMES[st] == "INVALID_ARGUMENT" and "aligned" in gq.gqap_last_error()
    st = call(ctypes.byref(p8), fake, fake, fake, fake, fake, fake, None, float("nan"), fake, fake, fake, None, None,
              0, None)
    assert gq.STATUS_NAMES[st] == "INVALID_ARGUMENT"


def test_fp8_prefill_rejects_missing_rope_tensors(gq):
    p8 = gq.gqap_prefill_plan(baseline_fp8_prefill_desc(gq))
    fake = 1 << 20  # never dereferenced: validation fails first
    st = gq.lib().gqap_prefill_fp8(ctypes.byref(p8), fake, None, fake, fake, fake, fake, None, 1.0, 1.0, 1.0, fake,
                                   None, None, 0, None)
    assert gq.STATUS_NAMES[st] == "INVALID_ARGUMENT" and "q_rope" in gq.gqap_last_error()


# ---------------------------------------------------------------- chunked prefill planning

def baseline_chunk_desc(gq):
    """8 sequences, chunks of up to 512 tokens, up to 6656 keys; pool [464, 8, 64, 128]."""
    d = gq.ChunkDesc()
    d.batch, d.num_q_heads, d.num_kv_heads, d.head_dim = 8, 32, 8, 128
    d.block_size, d.max_blocks_per_seq, d.num_pool_blocks = 64, 104, 464
    d.total_q_tokens, d.max_q_len, d.max_kv_len, d.dtype = 4096, 512, 6656, gq.BF16
    d.q_stride_head, d.q_stride_token = 128, 128 * 32
    d.new_stride_head, d.new_stride_token = 128, 128 * 8
    d.out_stride_head, d.out_stride_token = 128, 128 * 32
    d.kv_stride_head, d.kv_stride_block = 64 * 128, 8 * 64 * 128
    d.block_table_stride = 104
    return d


def test_chunk_plan_baseline(gq):
    p = gq.gqap_chunk_plan(baseline_chunk_desc(gq))
    assert p.magic == gq.PLAN_MAGIC and p.ratio == 4 and p.q_tile_rows == 128 and p.q_tiles == 4
    assert p.workspace_bytes == 0


@pytest.mark.parametrize("Hq,Hk,max_q,Dr,splits,kernel,head_chunks", [
    (32, 8, 4, 0, 0, 5, 1),       # 4 tokens x 4 heads: one 16-column tile
    (32, 8, 5, 0, 0, 1, 0),       # 20 pairs: two tiles where one token takes one -> prefill kernel
    (32, 8, 1, 0, 0, 5, 1),
    (16, 16, 16, 0, 0, 5, 1),     # one head per KV head, 16 tokens
    (16, 2, 2, 0, 0, 5, 1),
    (16, 2, 3, 0, 0, 1, 0),
    (10, 2, 3, 0, 0, 5, 1),       # 15 pairs
    (64, 2, 1, 0, 0, 5, 2),       # 32 heads per KV head take two tiles, as in decode
    (64, 2, 2, 0, 0, 1, 0),
    (32, 8, 4, 0, 1, 1, 0),       # forced splits keep the prefill kernel
    (32, 8, 4, 0, 2, 1, 0),
    (16, 16, 2, 64, 0, 5, 1),     # MLA (rope cache): the rope workers, one tile per head
    (16, 16, 16, 64, 0, 5, 1),
    (16, 16, 17, 64, 0, 2, 0),    # 17 tokens of one head: two tiles -> the MLA prefill kernel
    (16, 16, 2, 64, 1, 2, 0),     # forced splits keep the prefill kernel
])
def test_chunk_plan_routes_short_chunks_to_the_decode_workers(gq, Hq, Hk, max_q, Dr, splits, kernel, head_chunks):
    d = baseline_chunk_desc(gq)
    d.num_q_heads, d.num_kv_heads, d.max_q_len, d.num_splits = Hq, Hk, max_q, splits
    d.q_stride_head, d.q_stride_token = 128 + Dr, (128 + Dr) * Hq
    d.new_stride_head, d.new_stride_token = 128, 128 * Hk
    d.out_stride_head, d.out_stride_token = 128, 128 * Hq
    d.kv_stride_block = Hk * 64 * 128
    if Dr:
        d.head_dim_rope, d.kr_new_stride_token, d.kr_stride_block = Dr, Dr, 64 * Dr
    p = gq.gqap_chunk_plan(d)
    assert (p.kernel, p.head_chunks) == (kernel, head_chunks)
    if kernel == 5:
        # the decode workers' workspace: prefix, then per piece one LSE and one row of 128
        # floats per (token, head) column of a tile
        pieces = d.batch * Hk * head_chunks + p.num_workers
        cols = min(16, max_q * (Hq // Hk))
        assert p.num_workers == 768 and p.num_splits == 1
        r256 = lambda x: (x + 255) // 256 * 256  # noqa: E731
        assert p.workspace_bytes == r256((d.batch + 1) * 4) + r256(pieces * cols * 4) + r256(pieces * cols * 128 * 4)
        d.kv_dtype = gq.FP8_E4M3FN
        assert gq.gqap_chunk_plan(d).kernel == 6
    else:
        assert p.num_workers == 0


def test_chunk_decode_route_needs_a_workspace_without_a_gpu(gq):
    """The decode workers' route refuses a missing, short or misaligned
    workspace before touching any pointer."""
    d = baseline_chunk_desc(gq)
    d.max_q_len = 4
    p = gq.gqap_chunk_plan(d)
    assert p.kernel == 5 and p.workspace_bytes > 0
    lib = gq.lib()
    for ws, nbytes in ((None, 0), (256, p.workspace_bytes - 1), (272, p.workspace_bytes)):
        st = lib.gqap_chunk_prefill(ctypes.byref(p), 16, 16, 16, None, 16, 16, 16, 1.0, 16, None, ws, nbytes, None)
        assert gq.STATUS_NAMES[st] == "INVALID_ARGUMENT", (ws, nbytes, gq.gqap_last_error())


@pytest.mark.parametrize("field,value,status", [
    ("head_dim", 64, "UNSUPPORTED"),
    ("block_size", 32, "UNSUPPORTED"),
    ("dtype", 0, "DTYPE"),
    ("num_kv_heads", 5, "INVALID_ARGUMENT"),
    ("max_kv_len", 104 * 64 + 1, "INVALID_ARGUMENT"),   # past Nblk * 64
    ("max_q_len", 7000, "INVALID_ARGUMENT"),            # more chunk tokens than keys
    ("kv_stride_head", 64 * 128 - 8, "INVALID_ARGUMENT"),
    ("new_stride_token", 100, "INVALID_ARGUMENT"),
    ("block_table_stride", 50, "INVALID_ARGUMENT"),
    ("batch", -1, "INVALID_ARGUMENT"),
    ("head_dim_rope", 32, "UNSUPPORTED"),
    ("head_dim_rope", 64, "INVALID_ARGUMENT"),          # no rope strides, and q rows too narrow
])
def test_chunk_plan_rejects(gq, field, value, status):
    d = baseline_chunk_desc(gq)
    setattr(d, field, value)
    got = gq.lib().gqap_chunk_plan(ctypes.byref(d), ctypes.byref(gq.ChunkPlan()))
    assert gq.STATUS_NAMES[got] == status, gq.gqap_last_error()


def test_chunk_plan_mla(gq):
    d = baseline_chunk_desc(gq)
    d.head_dim_rope = 64
    d.q_stride_head, d.q_stride_token = 192, 192 * 32
    d.kr_new_stride_token, d.kr_stride_block = 64, 64 * 64
    p = gq.gqap_chunk_plan(d)
    assert p.magic == gq.PLAN_MAGIC and p.kernel == 2
    d.kr_stride_block = 64 * 63
    with pytest.raises(gq.GqapError, match="rope strides"):
        gq.gqap_chunk_plan(d)


def test_chunk_validate_host(gq):
    import numpy as np
    d = baseline_chunk_desc(gq)
    d.batch, d.total_q_tokens = 2, 600
    p = gq.gqap_chunk_plan(d)
    bt = np.full((2, 104), -1, np.int32)
    bt[0, :3] = [5, 6, 7]        # 150 keys
    bt[1, :9] = np.arange(9)     # 513 keys
    cu = np.array([0, 100, 600], np.int32)
    kv = np.array([150, 513], np.int32)
    gq.gqap_chunk_validate_host(p, bt, cu, kv)
    for bad_cu, bad_kv, what in (([0, 100, 700], [150, 513], "passes T"),
                                 ([0, 100, 600], [90, 513], "fewer keys than chunk tokens"),
                                 ([0, 100, 99], [150, 513], "decreasing"),
                                 ([1, 100, 600], [150, 513], "not starting at 0"),
                                 ([0, 100, 600], [150, 6657], "past max_kv_len")):
        with pytest.raises(gq.GqapError):
            gq.gqap_chunk_validate_host(p, bt, np.array(bad_cu, np.int32), np.array(bad_kv, np.int32))
    bt[1, 8] = 464               # outside the pool
    with pytest.raises(gq.GqapError, match="outside the pool"):
        gq.gqap_chunk_validate_host(p, bt, cu, kv)


def test_chunk_calls_reject_bad_arguments_without_a_gpu(gq):
    p = gq.gqap_chunk_plan(baseline_chunk_desc(gq))
    st = gq.lib().gqap_chunk_prefill(ctypes.byref(p), None, None, None, None, None, None, None, 1.0, None,
                                     None, None, 0, None)
    assert gq.STATUS_NAMES[st] == "INVALID_ARGUMENT"
    st = gq.lib().gqap_append_kv(ctypes.byref(p), None, None, None, None, None, None, None, None, None, None)
    assert gq.STATUS_NAMES[st] == "INVALID_ARGUMENT"
    # a rope cache passed to a plan without rope
    st = gq.lib().gqap_chunk_prefill(ctypes.byref(p), 16, 16, 16, 16, 16, 16, 16, 1.0, 16, None, None, 0, None)
    assert gq.STATUS_NAMES[st] == "INVALID_ARGUMENT"
    st = gq.lib().gqap_chunk_prefill(ctypes.byref(gq.ChunkPlan()), 16, 16, 16, None, 16, 16, 16, 1.0, 16, None,
                                     None, 0, None)
    assert gq.STATUS_NAMES[st] == "INVALID_ARGUMENT"      # unplanned (magic 0)


def test_chunk_plan_fp8_cache(gq):
    """kv_dtype FP8_E4M3FN plans an fp8 cache (pool strides in bytes, which
    must keep 16-byte slabs); 0 and BF16 plan a bf16 cache; other values are
    DTYPE errors."""
    d = baseline_chunk_desc(gq)
    assert gq.gqap_chunk_plan(d).kernel == 1
    d.kv_dtype = gq.BF16
    assert gq.gqap_chunk_plan(d).kernel == 1
    d.kv_dtype = gq.FP8_E4M3FN
    assert gq.gqap_chunk_plan(d).kernel == 3
    d.kv_stride_block = 8 * 64 * 128 + 8      # 8 bytes past a 16-byte boundary for fp8 pages
    with pytest.raises(gq.GqapError, match="16-byte"):
        gq.gqap_chunk_plan(d)
    for bad in (gq.F16, 7):
        d = baseline_chunk_desc(gq)
        d.kv_dtype = bad
        got = gq.lib().gqap_chunk_plan(ctypes.byref(d), ctypes.byref(gq.ChunkPlan()))
        assert gq.STATUS_NAMES[got] == "DTYPE", gq.gqap_last_error()


def test_chunk_calls_check_the_cache_dtype_without_a_gpu(gq):
    """The bf16 calls refuse an fp8-cache plan and the fp8 calls a bf16 one,
    before touching any pointer; the fp8 calls refuse scales that are not
    finite and positive."""
    lib = gq.lib()
    p16 = gq.gqap_chunk_plan(baseline_chunk_desc(gq))
    d8 = baseline_chunk_desc(gq)
    d8.kv_dtype = gq.FP8_E4M3FN
    p8 = gq.gqap_chunk_plan(d8)
    st = lib.gqap_chunk_prefill(ctypes.byref(p8), 16, 16, 16, None, 16, 16, 16, 1.0, 16, None, None, 0, None)
    assert gq.STATUS_NAMES[st] == "DTYPE"
    st = lib.gqap_append_kv(ctypes.byref(p8), 16, 16, None, 16, 16, None, 16, 16, 16, None)
    assert gq.STATUS_NAMES[st] == "DTYPE"
    st = lib.gqap_chunk_prefill_fp8kv(ctypes.byref(p16), 16, 16, 16, None, 16, 16, 16, 1.0, 1.0, 1.0, 16, None,
                                      None, 0, None)
    assert gq.STATUS_NAMES[st] == "DTYPE"
    st = lib.gqap_append_kv_fp8(ctypes.byref(p16), 16, 16, None, 16, 16, None, 16, 16, 16, 1.0, 1.0, None)
    assert gq.STATUS_NAMES[st] == "DTYPE"
    for ks, vs in ((0.0, 1.0), (1.0, -2.0), (float("inf"), 1.0), (1.0, float("nan"))):
        st = lib.gqap_chunk_prefill_fp8kv(ctypes.byref(p8), 16, 16, 16, None, 16, 16, 16, 1.0, ks, vs, 16, None,
                                          None, 0, None)
        assert gq.STATUS_NAMES[st] == "INVALID_ARGUMENT", (ks, vs)
        st = lib.gqap_append_kv_fp8(ctypes.byref(p8), 16, 16, None, 16, 16, None, 16, 16, 16, ks, vs, None)
        assert gq.STATUS_NAMES[st] == "INVALID_ARGUMENT", (ks, vs)
    st = lib.gqap_append_kv_fp8(ctypes.byref(p8), None, None, None, None, None, None, None, None, None, 1.0, 1.0,
                                None)
    assert gq.STATUS_NAMES[st] == "INVALID_ARGUMENT"


def test_csr_conversion_rejects_bad_arguments_without_a_gpu(gq):
    lib = gq.lib()
    assert gq.STATUS_NAMES[lib.gqap_block_table_from_csr(16, 16, -1, 4, 4, 16, None)] == "INVALID_ARGUMENT"
    assert gq.STATUS_NAMES[lib.gqap_block_table_from_csr(16, 16, 2, 0, 4, 16, None)] == "INVALID_ARGUMENT"
    assert gq.STATUS_NAMES[lib.gqap_block_table_from_csr(16, 16, 2, 4, 3, 16, None)] == "INVALID_ARGUMENT"
    assert gq.STATUS_NAMES[lib.gqap_block_table_from_csr(None, 16, 2, 4, 4, 16, None)] == "INVALID_ARGUMENT"
    assert gq.STATUS_NAMES[lib.gqap_block_table_from_csr(18, 16, 2, 4, 4, 16, None)] == "INVALID_ARGUMENT"
    assert lib.gqap_block_table_from_csr(None, None, 0, 4, 4, None, None) == 0   # empty batch: nothing to do


# ---------------------------------------------------------------- key-axis splits

def test_prefill_plans_split_small_grids_only(gq):
    # 4 x 16 x 24 = 1536 workgroups fill the GPU: no split, no workspace
    p = gq.gqap_prefill_plan(baseline_prefill_desc(gq))
    assert p.num_splits == 1 and p.workspace_bytes == 0
    # one 2048-token sequence, 16 heads: 256 workgroups, one per compute unit -> no split
    d = baseline_prefill_desc(gq)
    d.batch, d.total_tokens, d.max_seq_len = 1, 2048, 2048
    assert gq.gqap_prefill_plan(d).num_splits == 1
    # 8 heads: 128 workgroups leave half the units idle -> 4 splits
    d.num_q_heads = d.num_kv_heads = 8
    d.q_stride_token, d.k_stride_token = 192 * 8, 128 * 8
    d.v_stride_token, d.out_stride_token = 128 * 8, 128 * 8
    p = gq.gqap_prefill_plan(d)
    assert p.num_splits == 4 and p.workspace_bytes == 4 * 2048 * 8 * 129 * 4
    # a tiny grid is capped at 4 splits, and by a quarter of the key tiles
    d.num_q_heads = d.num_kv_heads = 2
    d.q_stride_token, d.k_stride_token = 192 * 2, 128 * 2
    d.v_stride_token, d.out_stride_token = 128 * 2, 128 * 2
    assert gq.gqap_prefill_plan(d).num_splits == 4
    d.total_tokens = d.max_seq_len = 300          # 5 key tiles -> at most 1 split
    assert gq.gqap_prefill_plan(d).num_splits == 1


def test_prefill_plan_forced_splits(gq):
    d = baseline_prefill_desc(gq)
    d.num_splits = 3
    p = gq.gqap_prefill_plan(d)
    assert p.num_splits == 3 and p.workspace_bytes == 3 * 6584 * 16 * 129 * 4
    for bad in (-1, 17):
        d.num_splits = bad
        st = gq.lib().gqap_prefill_plan(ctypes.byref(d), ctypes.byref(gq.PrefillPlan()))
        assert gq.STATUS_NAMES[st] == "INVALID_ARGUMENT"


def test_chunk_plan_splits(gq):
    d = baseline_chunk_desc(gq)                    # 8 x 32 x 4 = 1024 workgroups
    assert gq.gqap_chunk_plan(d).num_splits == 1
    d.batch, d.num_q_heads, d.num_kv_heads = 4, 16, 16   # 4 x 16 x 4 = 256: one per unit -> 1
    d.q_stride_token, d.out_stride_token = 128 * 16, 128 * 16
    d.new_stride_token, d.kv_stride_block = 128 * 16, 16 * 64 * 128
    assert gq.gqap_chunk_plan(d).num_splits == 1
    d.batch = 1                                          # 1 x 16 x 4 = 64 -> 4 splits
    p = gq.gqap_chunk_plan(d)
    assert p.num_splits == 4 and p.workspace_bytes == 4 * 4096 * 16 * 129 * 4
    d.num_splits = 5
    assert gq.gqap_chunk_plan(d).num_splits == 5


def test_split_calls_require_the_workspace(gq):
    """A split plan refuses a missing, short or misaligned workspace before any
    device work (the other pointers are never looked at)."""
    d = baseline_prefill_desc(gq)
    d.num_splits = 2
    p = gq.gqap_prefill_plan(d)
    fake = 1 << 20
    call = gq.lib().gqap_prefill
    for ws, wsb in ((None, 0), (fake, p.workspace_bytes - 16), (fake + 8, p.workspace_bytes)):
        st = call(ctypes.byref(p), fake, fake, fake, fake, fake, None, 1.0, fake, None, ws, wsb, None)
        assert gq.STATUS_NAMES[st] == "INVALID_ARGUMENT" and "workspace" in gq.gqap_last_error()


# ---------------------------------------------------------------- launch-size limits

def test_plans_reject_launches_past_2_to_the_32_work_items(gq):
    """Every launch stays under 2^32 work-items: the decode combine (one wave
    per sequence and query head), the split merge (one wave per token and
    head) and the append (one work-item per 16 bytes of a token's K/V row)."""
    lib = gq.lib()
    d = baseline_decode_desc(gq)
    d.batch, d.num_q_heads, d.num_kv_heads = 65535, 1025, 1
    d.q_stride_batch = d.out_stride_batch = 1025 * 128
    d.kv_stride_block = 64 * 128
    st = lib.gqap_decode_plan(ctypes.byref(d), ctypes.byref(gq.DecodePlan()))
    assert gq.STATUS_NAMES[st] == "UNSUPPORTED" and "combine" in gq.gqap_last_error()
    d.num_q_heads = 1024                           # 65535 x 1024 x 64 < 2^32
    d.q_stride_batch = d.out_stride_batch = 1024 * 128
    assert gq.gqap_decode_plan(d).magic == gq.PLAN_MAGIC

    p = baseline_prefill_desc(gq)                  # 16 heads
    p.total_tokens = (1 << 22) + 1                 # T x 16 x 64 > 2^32 once the merge runs
    p.num_splits = 2
    st = lib.gqap_prefill_plan(ctypes.byref(p), ctypes.byref(gq.PrefillPlan()))
    assert gq.STATUS_NAMES[st] == "UNSUPPORTED" and "merge" in gq.gqap_last_error()
    p.num_splits = 1                               # no merge: accepted
    assert gq.gqap_prefill_plan(p).magic == gq.PLAN_MAGIC

    c = baseline_chunk_desc(gq)                    # Hk = 8: 16 work-items per (token, KV head)
    c.total_q_tokens = (1 << 25)                   # 2^25 x 8 x 16 = 2^32
    st = lib.gqap_chunk_plan(ctypes.byref(c), ctypes.byref(gq.ChunkPlan()))
    assert gq.STATUS_NAMES[st] == "UNSUPPORTED" and "append" in gq.gqap_last_error()
    c.total_q_tokens = (1 << 25) - 2
    assert gq.gqap_chunk_plan(c).magic == gq.PLAN_MAGIC

    # the CSR conversion: one work-item per table entry
    st = lib.gqap_block_table_from_csr(16, 16, 65536, 65536, 65536, 16, None)
    assert gq.STATUS_NAMES[st] == "UNSUPPORTED"


def test_plans_keep_one_query_tile_for_rows_past_the_capacity(gq):
    """A sequence longer than max_seq_len has its rows past the capacity
    cleared by the last query tile's workgroup, so a plan with batch > 0
    always has at least one query tile, even for max_seq_len = 0."""
    d = baseline_prefill_desc(gq)
    d.max_seq_len = 0
    p = gq.gqap_prefill_plan(d)
    assert p.q_tiles == 1 and p.num_splits == 1
    d.batch = 0
    assert gq.gqap_prefill_plan(d).q_tiles == 0
    c = baseline_chunk_desc(gq)
    c.max_q_len = 0
    assert gq.gqap_chunk_plan(c).q_tiles == 1


def test_noalloc_decode_rejects_a_plan_past_its_scratch_without_a_gpu(gq):
    """The allocation-free decode checks the plan's workspace against its fixed
    scratch before any device call."""
    d = baseline_decode_desc(gq)
    d.num_workers = 20000                        # 20000+ partial slots of 4 x 128 floats: past 32 MiB
    p = gq.gqap_decode_plan(d)
    assert p.workspace_bytes > gq.NOALLOC_SCRATCH_BYTES
    st = gq.lib().gqap_paged_decode_noalloc(ctypes.byref(p), 16, 16, 16, 16, 16, 1.0, 1.0, 1.0, 16, None, None)
    assert gq.STATUS_NAMES[st] == "UNSUPPORTED" and "workspace" in gq.gqap_last_error()
    st = gq.lib().gqap_paged_decode_noalloc(ctypes.byref(gq.DecodePlan()), 16, 16, 16, 16, 16, 1.0, 1.0, 1.0, 16,
                                            None, None)
    assert gq.STATUS_NAMES[st] == "INVALID_ARGUMENT"
    assert gq.NOALLOC_SCRATCH_BYTES == 32 << 20
    text = open(HEADER).read()
    assert "#define GQAP_NOALLOC_SCRATCH_BYTES (32u << 20)" in text


def test_rope_fp8_prefill_rejects_bad_arguments_without_a_gpu(gq):
    """gqap_prefill_rope_fp8 validates before any device call: a plan of the
    wrong dtype, one without the rope part, a rope stride that is not a
    multiple of 16 bytes, null pointers."""
    lib = gq.lib()
    fake = 1 << 20
    call = lambda p, kr=fake, krs=fake: lib.gqap_prefill_rope_fp8(ctypes.byref(p), fake, fake, fake, kr, krs, fake,
                                                                   None, 0.1, fake, None, None, 0, None)
    d = baseline_prefill_desc(gq)
    d.kr_stride_token = 72                      # 72 bytes: not a multiple of 16
    p = gq.gqap_prefill_plan(d)
    assert gq.STATUS_NAMES[call(p)] == "INVALID_ARGUMENT" and "stride" in gq.gqap_last_error()
    d.kr_stride_token = 64
    p = gq.gqap_prefill_plan(d)
    assert gq.STATUS_NAMES[call(p, krs=None)] == "INVALID_ARGUMENT"
    assert gq.STATUS_NAMES[call(p, kr=None)] == "INVALID_ARGUMENT"
    assert gq.STATUS_NAMES[call(gq.gqap_prefill_plan(baseline_prefill_desc(gq, mla=False)))] == "INVALID_ARGUMENT"
    f = baseline_fp8_prefill_desc(gq)
    assert gq.STATUS_NAMES[call(gq.gqap_prefill_plan(f))] == "DTYPE"
