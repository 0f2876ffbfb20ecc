"""Generated cases on the device: move a case's storage bits to device tensors,
plan it through the library's C ABI and run it.  Argument marshalling only:
no attention arithmetic happens here (the kernels behind the C ABI do it).
Used by the GPU tests and by bench.py."""
from __future__ import annotations

import numpy as np
import torch

import gqa_attention_paged_amd as gq


def bits_to_tensor(x: np.ndarray, tag: str) -> torch.Tensor:
    if tag == "f32":
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if tag == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    if tag == "e4m3fn":
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint8)).view(torch.float8_e4m3fn)
    raise ValueError(tag)


def tensor_to_f64(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        bits = t.view(torch.int16).numpy().view(np.uint16)
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return t.numpy().astype(np.float64)


class DeviceDecode:
    """A decode case resident on the device plus a plan for it."""

    def __init__(self, case, num_workers: int = 0, device: str = "cuda", max_seq_len: int | None = None):
        self.case = case
        self.q = bits_to_tensor(case.q, case.q_dtype).to(device)
        self.k = bits_to_tensor(case.k_pool, case.kv_dtype).to(device)
        self.v = bits_to_tensor(case.v_pool, case.kv_dtype).to(device)
        self.bt = torch.from_numpy(np.ascontiguousarray(case.block_table, dtype=np.int32)).to(device)
        self.sl = torch.from_numpy(np.ascontiguousarray(case.seq_lens, dtype=np.int32)).to(device)
        self.out = torch.empty_like(self.q)
        self.lse = torch.empty((case.B, case.Hq), dtype=torch.float32, device=device)
        max_len = max(1, int(case.seq_lens.max())) if case.B else 1
        if max_seq_len is not None:
            max_len = max_seq_len
        self.desc = gq.decode_desc(self.q, self.k, self.bt, max_seq_len=max_len, out=self.out,
                                   num_workers=num_workers)
        self.plan = gq.gqap_decode_plan(self.desc)
        self.ws = torch.empty(max(256, self.plan.workspace_bytes), dtype=torch.uint8, device=device)

    def run(self, stream=None):
        c = self.case
        gq.gqap_paged_decode(self.plan, self.q, self.k, self.v, self.bt, self.sl, c.scale, c.k_scale, c.v_scale,
                             self.out, self.lse, self.ws, self.plan.workspace_bytes, stream=stream)
        return self.out, self.lse

    def results(self):
        torch.cuda.synchronize()
        return tensor_to_f64(self.out), self.lse.detach().cpu().numpy().astype(np.float64)


class DevicePrefill:
    """A ragged prefill case resident on the device plus a plan for it (and
    the workspace the plan asks for)."""

    def __init__(self, case, device: str = "cuda", num_splits: int = 0, max_seq_len: int | None = None):
        self.case = case
        self.fp8 = case.dtype == "e4m3fn"   # q holds the nope codes, q_rope the bf16 rope part
        self.q = bits_to_tensor(case.q, case.dtype).to(device)
        self.qr = bits_to_tensor(case.q_rope, "bf16").to(device) if case.q_rope is not None else None
        self.k = bits_to_tensor(case.k, case.dtype).to(device)
        self.v = bits_to_tensor(case.v, "bf16").to(device)
        # the shared rope key: bf16, or e4m3fn codes with one scale per row
        self.rope8 = getattr(case, "rope_dtype", "bf16") == "e4m3fn"
        self.kr = (bits_to_tensor(case.k_rope, "e4m3fn" if self.rope8 else "bf16").to(device)
                   if case.k_rope is not None else None)
        if self.rope8:
            self.krs = torch.from_numpy(np.ascontiguousarray(case.k_rope_scale, dtype=np.float32)).to(device)
        # fp8 with one scale per row of a head: [T, Hq] and [T, Hk] float32 arrays on the device
        self.blockwise = self.fp8 and np.ndim(case.q_scale) > 0
        if self.blockwise:
            self.qsc = torch.from_numpy(np.ascontiguousarray(case.q_scale, dtype=np.float32)).to(device)
            self.ksc = torch.from_numpy(np.ascontiguousarray(case.k_scale, dtype=np.float32)).to(device)
        self.cu = torch.from_numpy(np.ascontiguousarray(case.cu_seqlens, dtype=np.int32)).to(device)
        self.mask = (torch.from_numpy(np.ascontiguousarray(case.block_mask, dtype=np.uint8)).to(device)
                     if case.block_mask is not None else None)
        T = case.T
        self.out = torch.empty((T, case.Hq, case.D_v), dtype=torch.bfloat16, device=device)
        self.lse = torch.empty((T, case.Hq), dtype=torch.float32, device=device)
        max_len = max(1, int(case.seq_lens.max())) if case.B else 1
        if max_seq_len is not None:
            max_len = max_seq_len
        self.desc = gq.prefill_desc(self.q, self.k, self.v, self.kr, batch=case.B, max_seq_len=max_len,
                                    block_mask=self.mask, out=self.out, q_rope=self.qr, num_splits=num_splits)
        self.plan = gq.gqap_prefill_plan(self.desc)
        self.ws = torch.empty(max(256, self.plan.workspace_bytes), dtype=torch.uint8, device=device)

    def run(self, stream=None):
        ws, wsb = self.ws, self.plan.workspace_bytes
        if self.rope8:
            gq.gqap_prefill_rope_fp8(self.plan, self.q, self.k, self.v, self.kr, self.krs, self.cu, self.mask,
                                     self.case.scale, self.out, self.lse, ws, wsb, stream=stream)
        elif self.blockwise:
            gq.gqap_prefill_fp8_blockwise(self.plan, self.q, self.qr, self.k, self.v, self.kr, self.cu, self.mask,
                                          self.case.scale, self.qsc, self.ksc, self.out, self.lse, ws, wsb,
                                          stream=stream)
        elif self.fp8:
            gq.gqap_prefill_fp8(self.plan, self.q, self.qr, self.k, self.v, self.kr, self.cu, self.mask,
                                self.case.scale, self.case.q_scale, self.case.k_scale, self.out, self.lse, ws, wsb,
                                stream=stream)
        else:
            gq.gqap_prefill(self.plan, self.q, self.k, self.v, self.kr, self.cu, self.mask, self.case.scale,
                            self.out, self.lse, ws, wsb, stream=stream)
        return self.out, self.lse

    def results(self):
        torch.cuda.synchronize()
        return tensor_to_f64(self.out), self.lse.detach().cpu().numpy().astype(np.float64)


class DeviceChunk:
    """A chunked-prefill case on the device (cache with the prefixes filled)
    plus a plan for it."""

    def __init__(self, case, device: str = "cuda", num_splits: int = 0, max_q_len: int | None = None,
                 max_kv_len: int | None = None, validate: bool = True):
        self.case = case
        self.q = bits_to_tensor(case.q, "bf16").to(device)
        self.k_new = bits_to_tensor(case.k_new, "bf16").to(device)
        self.v_new = bits_to_tensor(case.v_new, "bf16").to(device)
        self.fp8 = getattr(case, "kv_dtype", "bf16") == "e4m3fn"   # fp8 cache with per-tensor scales
        pool_tag = "e4m3fn" if self.fp8 else "bf16"
        self.k_pool = bits_to_tensor(case.k_pool, pool_tag).to(device)
        self.v_pool = bits_to_tensor(case.v_pool, pool_tag).to(device)
        self.kr_new = bits_to_tensor(case.kr_new, "bf16").to(device) if case.kr_new is not None else None
        self.kr_pool = bits_to_tensor(case.kr_pool, "bf16").to(device) if case.kr_pool is not None else None
        self.bt = torch.from_numpy(np.ascontiguousarray(case.block_table, dtype=np.int32)).to(device)
        self.cu = torch.from_numpy(np.ascontiguousarray(case.cu_seqlens_q, dtype=np.int32)).to(device)
        self.kvl = torch.from_numpy(np.ascontiguousarray(case.kv_lens, dtype=np.int32)).to(device)
        T = case.T
        self.out = torch.empty((T, case.Hq, case.D), dtype=torch.bfloat16, device=device)
        self.lse = torch.empty((T, case.Hq), dtype=torch.float32, device=device)
        max_q = max(1, int(case.q_lens.max())) if case.B else 1
        max_kv = max(max_q, int(case.kv_lens.max())) if case.B else 1
        if max_q_len is not None:
            max_q = max_q_len
        if max_kv_len is not None:
            max_kv = max_kv_len
        self.desc = gq.chunk_desc(self.q, self.k_new, self.k_pool, self.bt, batch=case.B, max_q_len=max_q,
                                  max_kv_len=max_kv, out=self.out, k_rope_new=self.kr_new, kr_pool=self.kr_pool,
                                  num_splits=num_splits)
        self.plan = gq.gqap_chunk_plan(self.desc)
        self.ws = torch.empty(max(256, self.plan.workspace_bytes), dtype=torch.uint8, device=device)
        if validate:
            gq.gqap_chunk_validate_host(self.plan, case.block_table, case.cu_seqlens_q, case.kv_lens)

    def append(self, stream=None):
        if self.fp8:
            gq.gqap_append_kv_fp8(self.plan, self.k_new, self.v_new, self.kr_new, self.k_pool, self.v_pool,
                                  self.kr_pool, self.bt, self.cu, self.kvl, self.case.k_scale, self.case.v_scale,
                                  stream=stream)
            return
        gq.gqap_append_kv(self.plan, self.k_new, self.v_new, self.kr_new, self.k_pool, self.v_pool, self.kr_pool,
                          self.bt, self.cu, self.kvl, stream=stream)

    def run(self, stream=None):
        if self.fp8:
            gq.gqap_chunk_prefill_fp8kv(self.plan, self.q, self.k_pool, self.v_pool, self.kr_pool, self.bt, self.cu,
                                        self.kvl, self.case.scale, self.case.k_scale, self.case.v_scale, self.out,
                                        self.lse, self.ws, self.plan.workspace_bytes, stream=stream)
            return self.out, self.lse
        gq.gqap_chunk_prefill(self.plan, self.q, self.k_pool, self.v_pool, self.kr_pool, self.bt, self.cu,
                              self.kvl, self.case.scale, self.out, self.lse, self.ws, self.plan.workspace_bytes,
                              stream=stream)
        return self.out, self.lse

    def results(self):
        torch.cuda.synchronize()
        return tensor_to_f64(self.out), self.lse.detach().cpu().numpy().astype(np.float64)

    def pools_bits(self):
        """(k, v) pools as bf16 bits (uint8 codes for an fp8 cache), plus the rope pool for MLA cases."""
        torch.cuda.synchronize()
        bits = lambda t: t.detach().cpu().view(torch.int16).numpy().view(np.uint16)
        codes = lambda t: t.detach().cpu().view(torch.uint8).numpy()
        kv = codes if self.fp8 else bits
        if self.kr_pool is None:
            return kv(self.k_pool), kv(self.v_pool)
        return kv(self.k_pool), kv(self.v_pool), bits(self.kr_pool)
