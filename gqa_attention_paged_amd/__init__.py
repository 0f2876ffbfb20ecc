"""Python binding of libgqap.so (paged GQA decode + ragged MLA prefill on gfx950).

Argument marshalling only: every computation runs in the HIP kernels behind
the C ABI declared in include/gqap.h.  The functions below carry the C names;
device buffers are passed as torch tensors (or raw integer addresses) and the
stream defaults to torch's current stream.  There is no fallback: if the
shared library is missing, importing this package raises ImportError.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libgqap.so")

GQAP_OK = 0
GQAP_ERR_INVALID_ARGUMENT = 1
GQAP_ERR_DTYPE = 2
GQAP_ERR_UNSUPPORTED = 3
GQAP_ERR_HIP = 4
STATUS_NAMES = {0: "OK", 1: "INVALID_ARGUMENT", 2: "DTYPE", 3: "UNSUPPORTED", 4: "HIP"}

F32, BF16, FP8_E4M3FN, F16 = 0, 1, 2, 3
BLOCK_SIZE = 64
NOALLOC_SCRATCH_BYTES = 32 << 20   # GQAP_NOALLOC_SCRATCH_BYTES
PLAN_MAGIC = 0x47514150

C_FUNCTIONS = (
    "gqap_decode_plan", "gqap_decode_validate_host", "gqap_paged_decode", "gqap_paged_decode_noalloc",
    "gqap_debug_gather_kv",
    "gqap_prefill_plan", "gqap_prefill", "gqap_prefill_fp8", "gqap_prefill_fp8_blockwise",
    "gqap_prefill_rope_fp8", "gqap_chunk_plan",
    "gqap_chunk_validate_host", "gqap_append_kv", "gqap_chunk_prefill", "gqap_append_kv_fp8",
    "gqap_chunk_prefill_fp8kv", "gqap_block_table_from_csr", "gqap_last_error", "gqap_version",
)


class GqapError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"gqap status {STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class DecodeDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("block_size", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
        ("num_pool_blocks", ctypes.c_int32), ("max_seq_len", ctypes.c_int32), ("q_dtype", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("q_stride_batch", ctypes.c_int64), ("q_stride_head", ctypes.c_int64),
        ("out_stride_batch", ctypes.c_int64), ("out_stride_head", ctypes.c_int64),
        ("kv_stride_block", ctypes.c_int64), ("kv_stride_head", ctypes.c_int64),
        ("block_table_stride", ctypes.c_int64),
        ("num_workers", ctypes.c_int32), ("num_cus", ctypes.c_int32),
    ]


class DecodePlan(ctypes.Structure):
    _fields_ = [
        ("desc", DecodeDesc), ("num_workers", ctypes.c_int32), ("ratio", ctypes.c_int32),
        ("head_chunks", ctypes.c_int32), ("max_pieces", ctypes.c_int32), ("workspace_bytes", ctypes.c_uint64),
        ("magic", ctypes.c_uint32), ("kernel", ctypes.c_uint32),
    ]


class PrefillDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("head_dim_qk", ctypes.c_int32), ("head_dim_rope", ctypes.c_int32), ("head_dim_v", ctypes.c_int32),
        ("total_tokens", ctypes.c_int32), ("max_seq_len", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("causal", ctypes.c_int32), ("has_block_mask", ctypes.c_int32), ("mask_blocks", ctypes.c_int32),
        ("q_stride_token", ctypes.c_int64), ("q_stride_head", ctypes.c_int64),
        ("k_stride_token", ctypes.c_int64), ("k_stride_head", ctypes.c_int64),
        ("v_stride_token", ctypes.c_int64), ("v_stride_head", ctypes.c_int64),
        ("kr_stride_token", ctypes.c_int64),
        ("out_stride_token", ctypes.c_int64), ("out_stride_head", ctypes.c_int64),
        ("num_cus", ctypes.c_int32), ("num_splits", ctypes.c_int32),
        ("qr_stride_token", ctypes.c_int64), ("qr_stride_head", ctypes.c_int64),
    ]


class PrefillPlan(ctypes.Structure):
    _fields_ = [
        ("desc", PrefillDesc), ("ratio", ctypes.c_int32), ("q_tiles", ctypes.c_int32),
        ("q_tile_rows", ctypes.c_int32), ("kernel", ctypes.c_int32), ("workspace_bytes", ctypes.c_uint64),
        ("magic", ctypes.c_uint32), ("num_splits", ctypes.c_uint32),
    ]


class ChunkDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("block_size", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
        ("num_pool_blocks", ctypes.c_int32), ("total_q_tokens", ctypes.c_int32), ("max_q_len", ctypes.c_int32),
        ("max_kv_len", ctypes.c_int32), ("dtype", ctypes.c_int32), ("head_dim_rope", ctypes.c_int32),
        ("q_stride_token", ctypes.c_int64), ("q_stride_head", ctypes.c_int64),
        ("new_stride_token", ctypes.c_int64), ("new_stride_head", ctypes.c_int64),
        ("out_stride_token", ctypes.c_int64), ("out_stride_head", ctypes.c_int64),
        ("kv_stride_block", ctypes.c_int64), ("kv_stride_head", ctypes.c_int64),
        ("block_table_stride", ctypes.c_int64),
        ("kr_new_stride_token", ctypes.c_int64), ("kr_stride_block", ctypes.c_int64),
        ("num_splits", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
    ]


class ChunkPlan(ctypes.Structure):
    _fields_ = [
        ("desc", ChunkDesc), ("ratio", ctypes.c_int32), ("q_tiles", ctypes.c_int32),
        ("q_tile_rows", ctypes.c_int32), ("kernel", ctypes.c_int32), ("workspace_bytes", ctypes.c_uint64),
        ("magic", ctypes.c_uint32), ("num_splits", ctypes.c_uint32),
        ("num_workers", ctypes.c_int32), ("head_chunks", ctypes.c_int32),
    ]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run `python __graft_entry__.py` (build()) first")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, f32, u64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_uint64
    st = ctypes.c_int
    lib.gqap_decode_plan.argtypes = [ctypes.POINTER(DecodeDesc), ctypes.POINTER(DecodePlan)]
    lib.gqap_decode_plan.restype = st
    lib.gqap_decode_validate_host.argtypes = [ctypes.POINTER(DecodePlan), vp, vp]
    lib.gqap_decode_validate_host.restype = st
    lib.gqap_paged_decode.argtypes = [ctypes.POINTER(DecodePlan), vp, vp, vp, vp, vp, f32, f32, f32, vp, vp, vp,
                                      u64, vp]
    lib.gqap_paged_decode.restype = st
    lib.gqap_paged_decode_noalloc.argtypes = [ctypes.POINTER(DecodePlan), vp, vp, vp, vp, vp, f32, f32, f32, vp, vp,
                                              vp]
    lib.gqap_paged_decode_noalloc.restype = st
    lib.gqap_debug_gather_kv.argtypes = [ctypes.POINTER(DecodePlan), vp, vp, vp, i32, i32, i32, vp, vp]
    lib.gqap_debug_gather_kv.restype = st
    lib.gqap_prefill_plan.argtypes = [ctypes.POINTER(PrefillDesc), ctypes.POINTER(PrefillPlan)]
    lib.gqap_prefill_plan.restype = st
    lib.gqap_prefill.argtypes = [ctypes.POINTER(PrefillPlan), vp, vp, vp, vp, vp, vp, f32, vp, vp, vp, u64, vp]
    lib.gqap_prefill.restype = st
    lib.gqap_prefill_fp8.argtypes = [ctypes.POINTER(PrefillPlan), vp, vp, vp, vp, vp, vp, vp, f32, f32, f32, vp, vp,
                                     vp, u64, vp]
    lib.gqap_prefill_fp8.restype = st
    lib.gqap_prefill_fp8_blockwise.argtypes = [ctypes.POINTER(PrefillPlan), vp, vp, vp, vp, vp, vp, vp, f32, vp, vp,
                                               vp, vp, vp, u64, vp]
    lib.gqap_prefill_fp8_blockwise.restype = st
    lib.gqap_prefill_rope_fp8.argtypes = [ctypes.POINTER(PrefillPlan), vp, vp, vp, vp, vp, vp, vp, f32, vp, vp, vp,
                                          u64, vp]
    lib.gqap_prefill_rope_fp8.restype = st
    lib.gqap_chunk_plan.argtypes = [ctypes.POINTER(ChunkDesc), ctypes.POINTER(ChunkPlan)]
    lib.gqap_chunk_plan.restype = st
    lib.gqap_chunk_validate_host.argtypes = [ctypes.POINTER(ChunkPlan), vp, vp, vp]
    lib.gqap_chunk_validate_host.restype = st
    lib.gqap_append_kv.argtypes = [ctypes.POINTER(ChunkPlan), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.gqap_append_kv.restype = st
    lib.gqap_chunk_prefill.argtypes = [ctypes.POINTER(ChunkPlan), vp, vp, vp, vp, vp, vp, vp, f32, vp, vp, vp, u64,
                                       vp]
    lib.gqap_chunk_prefill.restype = st
    lib.gqap_append_kv_fp8.argtypes = [ctypes.POINTER(ChunkPlan), vp, vp, vp, vp, vp, vp, vp, vp, vp, f32, f32, vp]
    lib.gqap_append_kv_fp8.restype = st
    lib.gqap_chunk_prefill_fp8kv.argtypes = [ctypes.POINTER(ChunkPlan), vp, vp, vp, vp, vp, vp, vp, f32, f32, f32, vp,
                                             vp, vp, u64, vp]
    lib.gqap_chunk_prefill_fp8kv.restype = st
    lib.gqap_block_table_from_csr.argtypes = [vp, vp, i32, i32, ctypes.c_int64, vp, vp]
    lib.gqap_block_table_from_csr.restype = st
    lib.gqap_last_error.argtypes = []
    lib.gqap_last_error.restype = ctypes.c_char_p
    lib.gqap_version.argtypes = []
    lib.gqap_version.restype = ctypes.c_char_p
    return lib


_lib = _load()


def lib() -> ctypes.CDLL:
    return _lib


def _check(status: int) -> None:
    if status != GQAP_OK:
        raise GqapError(status, _lib.gqap_last_error().decode())


def _ptr(x) -> Optional[int]:
    """Device address of a tensor (or an int / None passed through)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ------------------------------------------------------------------ C names

def gqap_version() -> str:
    return _lib.gqap_version().decode()


def gqap_last_error() -> str:
    return _lib.gqap_last_error().decode()


def gqap_decode_plan(desc: DecodeDesc) -> DecodePlan:
    plan = DecodePlan()
    _check(_lib.gqap_decode_plan(ctypes.byref(desc), ctypes.byref(plan)))
    return plan


def gqap_decode_validate_host(plan: DecodePlan, block_table_host, seq_lens_host) -> None:
    """Host arrays (numpy int32, C-contiguous with the plan's row stride)."""
    import numpy as np
    bt = np.ascontiguousarray(block_table_host, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens_host, dtype=np.int32)
    _check(_lib.gqap_decode_validate_host(ctypes.byref(plan), bt.ctypes.data, sl.ctypes.data))


def gqap_paged_decode(plan: DecodePlan, q, k_pool, v_pool, block_table, seq_lens, scale: float,
                      k_scale: float, v_scale: float, out, lse=None, workspace=None,
                      workspace_bytes: Optional[int] = None, stream=None) -> None:
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.gqap_paged_decode(ctypes.byref(plan), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table),
                                  _ptr(seq_lens), scale, k_scale, v_scale, _ptr(out), _ptr(lse), _ptr(workspace),
                                  workspace_bytes, _stream(stream)))


def gqap_paged_decode_noalloc(plan: DecodePlan, q, k_pool, v_pool, block_table, seq_lens, scale: float,
                              k_scale: float, v_scale: float, out, lse=None, stream=None) -> None:
    _check(_lib.gqap_paged_decode_noalloc(ctypes.byref(plan), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                          _ptr(block_table), _ptr(seq_lens), scale, k_scale, v_scale, _ptr(out),
                                          _ptr(lse), _stream(stream)))


def gqap_debug_gather_kv(plan: DecodePlan, pool, block_table, seq_lens, b: int, kv_head: int, num_rows: int,
                         dst, stream=None) -> None:
    _check(_lib.gqap_debug_gather_kv(ctypes.byref(plan), _ptr(pool), _ptr(block_table), _ptr(seq_lens), b,
                                     kv_head, num_rows, _ptr(dst), _stream(stream)))


def gqap_prefill_plan(desc: PrefillDesc) -> PrefillPlan:
    plan = PrefillPlan()
    _check(_lib.gqap_prefill_plan(ctypes.byref(desc), ctypes.byref(plan)))
    return plan


def gqap_prefill(plan: PrefillPlan, q, k, v, k_rope, cu_seqlens, block_mask, scale: float, out, lse=None,
                 workspace=None, workspace_bytes: Optional[int] = None, stream=None) -> None:
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.gqap_prefill(ctypes.byref(plan), _ptr(q), _ptr(k), _ptr(v), _ptr(k_rope), _ptr(cu_seqlens),
                             _ptr(block_mask), scale, _ptr(out), _ptr(lse), _ptr(workspace), workspace_bytes,
                             _stream(stream)))


def gqap_prefill_fp8(plan: PrefillPlan, q_nope, q_rope, k, v, k_rope, cu_seqlens, block_mask, scale: float,
                     q_scale: float, k_scale: float, out, lse=None, workspace=None,
                     workspace_bytes: Optional[int] = None, stream=None) -> None:
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.gqap_prefill_fp8(ctypes.byref(plan), _ptr(q_nope), _ptr(q_rope), _ptr(k), _ptr(v), _ptr(k_rope),
                                 _ptr(cu_seqlens), _ptr(block_mask), scale, q_scale, k_scale, _ptr(out), _ptr(lse),
                                 _ptr(workspace), workspace_bytes, _stream(stream)))


def gqap_prefill_fp8_blockwise(plan: PrefillPlan, q_nope, q_rope, k, v, k_rope, cu_seqlens, block_mask,
                               scale: float, q_scales, k_scales, out, lse=None, workspace=None,
                               workspace_bytes: Optional[int] = None, stream=None) -> None:
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.gqap_prefill_fp8_blockwise(ctypes.byref(plan), _ptr(q_nope), _ptr(q_rope), _ptr(k), _ptr(v),
                                           _ptr(k_rope), _ptr(cu_seqlens), _ptr(block_mask), scale, _ptr(q_scales),
                                           _ptr(k_scales), _ptr(out), _ptr(lse), _ptr(workspace), workspace_bytes,
                                           _stream(stream)))


def gqap_prefill_rope_fp8(plan: PrefillPlan, q, k, v, k_rope, k_rope_scales, cu_seqlens, block_mask, scale: float,
                          out, lse=None, workspace=None, workspace_bytes: Optional[int] = None, stream=None) -> None:
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.gqap_prefill_rope_fp8(ctypes.byref(plan), _ptr(q), _ptr(k), _ptr(v), _ptr(k_rope),
                                      _ptr(k_rope_scales), _ptr(cu_seqlens), _ptr(block_mask), scale, _ptr(out),
                                      _ptr(lse), _ptr(workspace), workspace_bytes, _stream(stream)))


def gqap_chunk_plan(desc: ChunkDesc) -> ChunkPlan:
    plan = ChunkPlan()
    _check(_lib.gqap_chunk_plan(ctypes.byref(desc), ctypes.byref(plan)))
    return plan


def gqap_chunk_validate_host(plan: ChunkPlan, block_table_host, cu_seqlens_q_host, kv_lens_host) -> None:
    """Host arrays (numpy int32, C-contiguous with the plan's row stride)."""
    import numpy as np
    bt = np.ascontiguousarray(block_table_host, dtype=np.int32)
    cu = np.ascontiguousarray(cu_seqlens_q_host, dtype=np.int32)
    kl = np.ascontiguousarray(kv_lens_host, dtype=np.int32)
    _check(_lib.gqap_chunk_validate_host(ctypes.byref(plan), bt.ctypes.data, cu.ctypes.data, kl.ctypes.data))


def gqap_append_kv(plan: ChunkPlan, k_new, v_new, k_rope_new, k_pool, v_pool, kr_pool, block_table,
                   cu_seqlens_q, kv_lens, stream=None) -> None:
    _check(_lib.gqap_append_kv(ctypes.byref(plan), _ptr(k_new), _ptr(v_new), _ptr(k_rope_new), _ptr(k_pool),
                               _ptr(v_pool), _ptr(kr_pool), _ptr(block_table), _ptr(cu_seqlens_q), _ptr(kv_lens),
                               _stream(stream)))


def gqap_chunk_prefill(plan: ChunkPlan, q, k_pool, v_pool, kr_pool, block_table, cu_seqlens_q, kv_lens,
                       scale: float, out, lse=None, workspace=None, workspace_bytes: Optional[int] = None,
                       stream=None) -> None:
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.gqap_chunk_prefill(ctypes.byref(plan), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(kr_pool),
                                   _ptr(block_table), _ptr(cu_seqlens_q), _ptr(kv_lens), scale, _ptr(out),
                                   _ptr(lse), _ptr(workspace), workspace_bytes, _stream(stream)))


def gqap_append_kv_fp8(plan: ChunkPlan, k_new, v_new, k_rope_new, k_pool, v_pool, kr_pool, block_table,
                       cu_seqlens_q, kv_lens, k_scale: float, v_scale: float, stream=None) -> None:
    _check(_lib.gqap_append_kv_fp8(ctypes.byref(plan), _ptr(k_new), _ptr(v_new), _ptr(k_rope_new), _ptr(k_pool),
                                   _ptr(v_pool), _ptr(kr_pool), _ptr(block_table), _ptr(cu_seqlens_q),
                                   _ptr(kv_lens), k_scale, v_scale, _stream(stream)))


def gqap_chunk_prefill_fp8kv(plan: ChunkPlan, q, k_pool, v_pool, kr_pool, block_table, cu_seqlens_q, kv_lens,
                             scale: float, k_scale: float, v_scale: float, out, lse=None, workspace=None,
                             workspace_bytes: Optional[int] = None, stream=None) -> None:
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.gqap_chunk_prefill_fp8kv(ctypes.byref(plan), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(kr_pool),
                                         _ptr(block_table), _ptr(cu_seqlens_q), _ptr(kv_lens), scale, k_scale,
                                         v_scale, _ptr(out), _ptr(lse), _ptr(workspace), workspace_bytes,
                                         _stream(stream)))


def gqap_block_table_from_csr(kv_indices, kv_page_indptr, batch: int, max_blocks_per_seq: int, block_table,
                              block_table_stride: Optional[int] = None, stream=None) -> None:
    if block_table_stride is None:
        block_table_stride = block_table.stride(0)
    _check(_lib.gqap_block_table_from_csr(_ptr(kv_indices), _ptr(kv_page_indptr), batch, max_blocks_per_seq,
                                          block_table_stride, _ptr(block_table), _stream(stream)))


# ------------------------------------------------------------------ descriptors from tensors

_TORCH_DTYPE_TAG = {"torch.float32": F32, "torch.bfloat16": BF16, "torch.float8_e4m3fn": FP8_E4M3FN,
                    "torch.float16": F16}


def dtype_tag(t) -> int:
    key = str(t.dtype)
    if key not in _TORCH_DTYPE_TAG:
        raise GqapError(GQAP_ERR_DTYPE, f"tensor dtype {t.dtype} has no gqap dtype")
    return _TORCH_DTYPE_TAG[key]


def decode_desc(q, k_pool, block_table, max_seq_len: int, out=None, num_workers: int = 0,
                num_cus: int = 0) -> DecodeDesc:
    """Descriptor for q [B, Hq, D], pool [NB, Hk, 64, D], block_table [B, Nblk]."""
    B, Hq, D = q.shape
    NB, Hk, blk, Dk = k_pool.shape
    out = q if out is None else out
    d = DecodeDesc()
    d.batch, d.num_q_heads, d.num_kv_heads, d.head_dim = B, Hq, Hk, D
    d.block_size = blk
    d.max_blocks_per_seq = block_table.shape[1]
    d.num_pool_blocks = NB
    d.max_seq_len = max_seq_len
    d.q_dtype = dtype_tag(q)
    d.kv_dtype = dtype_tag(k_pool)
    d.q_stride_batch, d.q_stride_head = q.stride(0), q.stride(1)
    d.out_stride_batch, d.out_stride_head = out.stride(0), out.stride(1)
    d.kv_stride_block, d.kv_stride_head = k_pool.stride(0), k_pool.stride(1)
    d.block_table_stride = block_table.stride(0)
    d.num_workers = num_workers
    d.num_cus = num_cus
    return d


def prefill_desc(q, k, v, k_rope, batch: int, max_seq_len: int, block_mask=None, out=None,
                 num_cus: int = 0, q_rope=None, num_splits: int = 0) -> PrefillDesc:
    """Descriptor for ragged q [T, Hq, Dqk], k [T, Hk, Dn], v [T, Hk, Dv], k_rope [T, 1, Dr] or None.
    fp8: q is q_nope [T, Hq, Dn] (codes) and q_rope [T, Hq, Dr] the bf16 rope part, or None."""
    T, Hq, Dqk = q.shape
    if q_rope is not None:
        Dqk += q_rope.shape[2]
    Hk = k.shape[1]
    out = out if out is not None else v.new_empty((T, Hq, v.shape[2]))
    d = PrefillDesc()
    d.batch, d.num_q_heads, d.num_kv_heads = batch, Hq, Hk
    d.head_dim_qk = Dqk
    d.head_dim_rope = 0 if k_rope is None else k_rope.shape[2]
    d.head_dim_v = v.shape[2]
    d.total_tokens = T
    d.max_seq_len = max_seq_len
    d.dtype = dtype_tag(q)
    d.causal = 1
    d.has_block_mask = 0 if block_mask is None else 1
    d.mask_blocks = 0 if block_mask is None else block_mask.shape[1]
    d.q_stride_token, d.q_stride_head = q.stride(0), q.stride(1)
    d.k_stride_token, d.k_stride_head = k.stride(0), k.stride(1)
    d.v_stride_token, d.v_stride_head = v.stride(0), v.stride(1)
    d.kr_stride_token = 0 if k_rope is None else k_rope.stride(0)
    d.out_stride_token, d.out_stride_head = out.stride(0), out.stride(1)
    d.num_cus = num_cus
    d.num_splits = num_splits
    if q_rope is not None:
        d.qr_stride_token, d.qr_stride_head = q_rope.stride(0), q_rope.stride(1)
    return d


def chunk_desc(q, k_new, k_pool, block_table, batch: int, max_q_len: int, max_kv_len: int,
               out=None, k_rope_new=None, kr_pool=None, num_splits: int = 0) -> ChunkDesc:
    """Descriptor for q [T, Hq, D + Dr], k_new / v_new [T, Hk, D], pool [NB, Hk, 64, D],
    block_table [B, Nblk]; MLA: k_rope_new [T, 1, Dr], kr_pool [NB, 1, 64, Dr].
    A float8_e4m3fn pool makes an fp8 cache (kv_dtype FP8_E4M3FN)."""
    T, Hq, _ = q.shape
    NB, Hk, blk, D = k_pool.shape
    out = q if out is None else out
    d = ChunkDesc()
    d.batch, d.num_q_heads, d.num_kv_heads, d.head_dim = batch, Hq, Hk, D
    d.block_size = blk
    d.max_blocks_per_seq = block_table.shape[1]
    d.num_pool_blocks = NB
    d.total_q_tokens = T
    d.max_q_len = max_q_len
    d.max_kv_len = max_kv_len
    d.dtype = dtype_tag(q)
    d.q_stride_token, d.q_stride_head = q.stride(0), q.stride(1)
    d.new_stride_token, d.new_stride_head = k_new.stride(0), k_new.stride(1)
    d.out_stride_token, d.out_stride_head = out.stride(0), out.stride(1)
    d.kv_stride_block, d.kv_stride_head = k_pool.stride(0), k_pool.stride(1)
    d.kv_dtype = dtype_tag(k_pool)
    d.block_table_stride = block_table.stride(0)
    if kr_pool is not None:
        d.head_dim_rope = kr_pool.shape[3]
        d.kr_new_stride_token = k_rope_new.stride(0)
        d.kr_stride_block = kr_pool.stride(0)
    d.num_splits = num_splits
    return d
