"""Seeded synthetic inputs for paged GQA decode and ragged (MLA) prefill.

This module is shared by the CPU oracle tests, the GPU parity tests and the
benchmark.  It only *draws* inputs: lengths, block tables, normal values and
their rounding to the storage dtypes (bf16 by round-to-nearest-even, OCP fp8
e4m3fn by saturating round-to-nearest-even, both done by torch CPU casts).  It
holds none of the attention arithmetic: no gather, no dot products, no softmax.

Everything is returned as numpy arrays of *storage bits* plus a dtype tag:
  'f32'    -> float32 values
  'bf16'   -> uint16 bit patterns
  'e4m3fn' -> uint8 bit patterns
so that a consumer (the oracle or the device path) decides itself how to read
them.

Physical KV pool layout (FlashMLA tensor-shape reference, "Paged KV Cache"
diagram and "Prefill to Cache Mapping"): a shared pool [NB, Hk, 64, D]; the
logical token t of sequence b lives in pool block block_table[b, t // 64] at
row t % 64.  Slots past seq_len and pool blocks no sequence uses are filled with
NaN so that any read of them is visible in the output.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np
import torch

BLOCK = 64                      # paged-cache block size (always 64 on the pages)
BF16_NAN = np.uint16(0x7FC0)
E4M3FN_NAN = np.uint8(0x7F)
E4M3FN_MAX = 448.0
_CHUNK = 1 << 22


def _threads() -> int:
    try:
        import os
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except Exception:  # pragma: no cover
        return 4


def normal_f32(seed_seq: np.random.SeedSequence, n: int) -> np.ndarray:
    """n standard-normal float32 values, deterministic for a given SeedSequence.

    The array is cut into fixed chunks of 2**22 values, chunk i drawn from the
    i-th spawned child stream, so the result does not depend on the number of
    threads used to fill it."""
    out = np.empty(n, np.float32)
    nch = (n + _CHUNK - 1) // _CHUNK
    kids = seed_seq.spawn(nch)

    def fill(i: int) -> None:
        g = np.random.Generator(np.random.PCG64(kids[i]))
        s = i * _CHUNK
        e = min(n, s + _CHUNK)
        g.standard_normal(e - s, dtype=np.float32, out=out[s:e])

    if nch <= 1:
        for i in range(nch):
            fill(i)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nch)))
    return out


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 -> bf16 (torch CPU cast, round-to-nearest-even); return uint16 bits."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def to_e4m3fn_bits(x: np.ndarray, scale: float) -> np.ndarray:
    """Quantise x / scale to OCP fp8 e4m3fn bytes with saturation to +-448
    (scale a float, or an array that broadcasts against x).

    torch's cast rounds to nearest even but does not saturate (values >= 480
    become NaN), hence the clamp first."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if np.ndim(scale):  # one scale per block, broadcast against x
        t = (t / torch.from_numpy(np.ascontiguousarray(scale, dtype=np.float32))).clamp_(-E4M3FN_MAX, E4M3FN_MAX)
    else:
        t = (t / np.float32(scale)).clamp_(-E4M3FN_MAX, E4M3FN_MAX)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


# --------------------------------------------------------------------------
# Paged decode
# --------------------------------------------------------------------------

@dataclass
class DecodeCase:
    name: str
    B: int
    Hq: int
    Hk: int
    D: int
    q: np.ndarray            # [B, Hq, D] bits
    k_pool: np.ndarray       # [NB, Hk, 64, D] bits
    v_pool: np.ndarray       # [NB, Hk, 64, D] bits
    block_table: np.ndarray  # [B, Nblk] int32 (unused entries: -1 or a NaN block)
    seq_lens: np.ndarray     # [B] int32
    q_dtype: str
    kv_dtype: str
    scale: float
    k_scale: float = 1.0
    v_scale: float = 1.0
    meta: dict = field(default_factory=dict)

    @property
    def NB(self) -> int:
        return int(self.k_pool.shape[0])

    @property
    def Nblk(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.B else 0

    def kv_bytes(self) -> int:
        """Bytes of K and V rows the decode must read (valid rows only)."""
        esz = {"f32": 4, "bf16": 2, "e4m3fn": 1}[self.kv_dtype]
        return int(self.seq_lens.astype(np.int64).sum()) * self.Hk * self.D * 2 * esz


def _blocks_needed(seq_lens: np.ndarray) -> np.ndarray:
    return (seq_lens.astype(np.int64) + BLOCK - 1) // BLOCK


def make_decode_case(
    *,
    name: str,
    seed: int,
    B: int,
    Hq: int,
    Hk: int,
    D: int,
    q_dtype: str,
    kv_dtype: str,
    seq_lens: Optional[Sequence[int]] = None,
    len_range: Optional[tuple] = None,
    pool_blocks: Optional[int] = None,
    nblk: Optional[int] = None,
    injective_table: bool = False,
    scale: Optional[float] = None,
) -> DecodeCase:
    """Draw a paged decode problem.

    Draw order: seq_lens -> block_table permutation -> q -> k -> v.

    seq_lens: explicit list, or drawn uniformly from the inclusive len_range.
    Pool: by default exactly sum(ceil(L/64)) blocks; the logical blocks (b, j)
    in row-major order take a seeded permutation of the pool ids and unused
    table entries are -1.  With ``injective_table`` every one of the B*Nblk
    table entries takes a distinct pool id (a seeded injection into a pool of
    ``pool_blocks``), so padding entries point at real, NaN-filled blocks.
    """
    ss = np.random.SeedSequence(seed)
    s_len, s_tab, s_q, s_k, s_v = ss.spawn(5)
    if seq_lens is None:
        lo, hi = len_range
        seq_lens = np.random.Generator(np.random.PCG64(s_len)).integers(lo, hi + 1, size=B)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    assert seq_lens.shape == (B,)
    need = _blocks_needed(seq_lens)
    if nblk is None:
        nblk = max(1, int(need.max()) if B else 1)
    g_tab = np.random.Generator(np.random.PCG64(s_tab))
    if injective_table:
        NB = pool_blocks if pool_blocks is not None else B * nblk
        assert NB >= B * nblk
        perm = g_tab.permutation(NB)
        block_table = perm[: B * nblk].reshape(B, nblk).astype(np.int32)
        used = np.zeros(NB, bool)
        for b in range(B):
            used[block_table[b, : need[b]]] = True
    else:
        NB = int(need.sum()) if pool_blocks is None else pool_blocks
        assert NB >= int(need.sum())
        perm = g_tab.permutation(NB)
        block_table = np.full((B, nblk), -1, np.int32)
        k = 0
        for b in range(B):
            for j in range(int(need[b])):
                block_table[b, j] = perm[k]
                k += 1
        used = np.zeros(NB, bool)
        used[perm[:k]] = True

    if scale is None:
        scale = 1.0 / math.sqrt(D)

    qf = normal_f32(s_q, B * Hq * D).reshape(B, Hq, D)
    if q_dtype == "f32":
        q = qf
    elif q_dtype == "bf16":
        q = to_bf16_bits(qf)
    else:
        raise ValueError(q_dtype)

    pool_shape = (NB, Hk, BLOCK, D)
    n_pool = NB * Hk * BLOCK * D
    scales = {}
    pools = []
    for nm, s_x in (("k", s_k), ("v", s_v)):
        xf = normal_f32(s_x, n_pool).reshape(pool_shape)
        if kv_dtype == "f32":
            x = xf
            nan = np.float32("nan")
            scales[nm] = 1.0
        elif kv_dtype == "bf16":
            x = to_bf16_bits(xf)
            nan = BF16_NAN
            scales[nm] = 1.0
        elif kv_dtype == "e4m3fn":
            amax = float(np.abs(xf).max()) if n_pool else 1.0
            sc = float(np.float32(amax) / np.float32(E4M3FN_MAX))
            x = to_e4m3fn_bits(xf, sc)
            nan = E4M3FN_NAN
            scales[nm] = sc
        else:
            raise ValueError(kv_dtype)
        del xf
        # poison: unused blocks entirely, and the tail rows of each last block
        x[~used] = nan
        for b in range(B):
            L = int(seq_lens[b])
            if L % BLOCK and need[b] > 0:
                x[block_table[b, need[b] - 1], :, L % BLOCK:, :] = nan
        pools.append(x)

    return DecodeCase(
        name=name, B=B, Hq=Hq, Hk=Hk, D=D, q=q, k_pool=pools[0], v_pool=pools[1],
        block_table=block_table, seq_lens=seq_lens, q_dtype=q_dtype, kv_dtype=kv_dtype,
        scale=float(scale), k_scale=scales["k"], v_scale=scales["v"],
        meta={"seed": seed, "used_blocks": used},
    )


def decode_tiny_fp32(seed: int = 1001) -> DecodeCase:
    """B=2, Hq=8, Hk=4, D=64, seq_lens {100, 37}, Nblk=2, pool of 6 blocks with a
    seeded injective block_table, fp32, NaN in every unused slot."""
    return make_decode_case(name="decode_tiny_f32", seed=seed, B=2, Hq=8, Hk=4, D=64,
                            q_dtype="f32", kv_dtype="f32", seq_lens=[100, 37],
                            pool_blocks=6, nblk=2, injective_table=True)


def decode_gqa_bf16(seed: int = 1002, B: int = 64, len_range=(1024, 4096)) -> DecodeCase:
    """B=64, Hq=32, Hk=8, D=128, seq_lens ~ U{1024..4096}, bf16 q/K/V."""
    return make_decode_case(name="decode_gqa_bf16", seed=seed, B=B, Hq=32, Hk=8, D=128,
                            q_dtype="bf16", kv_dtype="bf16", len_range=len_range)


def decode_long_fp8(seed: int = 1004, B: int = 128, len_range=(4096, 8192)) -> DecodeCase:
    """B=128, Hq=64, Hk=8, D=128, seq_lens ~ U{4096..8192}, bf16 q, fp8 e4m3fn K/V
    with per-tensor scales amax/448."""
    return make_decode_case(name="decode_long_fp8", seed=seed, B=B, Hq=64, Hk=8, D=128,
                            q_dtype="bf16", kv_dtype="e4m3fn", len_range=len_range)


# --------------------------------------------------------------------------
# Ragged prefill
# --------------------------------------------------------------------------

@dataclass
class PrefillCase:
    name: str
    seq_lens: np.ndarray      # [B] int32
    cu_seqlens: np.ndarray    # [B+1] int32, [0, cumsum(seq_lens)]
    Hq: int
    Hk: int
    D_qk: int                 # width of a query head (nope + rope)
    D_rope: int               # width of the shared rope key (0 if none)
    D_v: int
    q: np.ndarray             # [T, Hq, D_qk] bf16 bits
    k: np.ndarray             # [T, Hk, D_qk - D_rope] bf16 bits
    v: np.ndarray             # [T, Hk, D_v] bf16 bits
    k_rope: Optional[np.ndarray]   # [T, 1, D_rope] bf16 bits, or None
    block_mask: Optional[np.ndarray]  # [B, nb, nb] uint8, or None
    scale: float
    dtype: str = "bf16"
    # dtype 'e4m3fn': q holds the nope part only, [T, Hq, D_nope] e4m3fn codes,
    # k [T, Hk, D_nope] e4m3fn codes, q_rope [T, Hq, D_rope] bf16 bits (None
    # without rope); q_scale / k_scale are the two tensors' scales (per tensor
    # or per row of a head).
    q_rope: Optional[np.ndarray] = None
    q_scale: object = 1.0     # float, or float32 [T, Hq] with blockwise scales
    k_scale: object = 1.0     # float, or float32 [T, Hk]
    # rope_dtype 'e4m3fn': k_rope holds e4m3fn codes [T, 1, D_rope] with one
    # float32 scale per row in k_rope_scale [T]; q, k and v stay bf16.
    rope_dtype: str = "bf16"
    k_rope_scale: Optional[np.ndarray] = None
    meta: dict = field(default_factory=dict)

    @property
    def B(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def T(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def D_nope(self) -> int:
        return self.D_qk - self.D_rope

    def visible_pairs(self) -> int:
        """Number of (query, key) pairs the causal (and block-sparse) mask lets through."""
        tot = 0
        for b in range(self.B):
            L = int(self.seq_lens[b])
            if self.block_mask is None:
                tot += L * (L + 1) // 2
                continue
            nb = (L + BLOCK - 1) // BLOCK
            for i in range(nb):
                rows = min(BLOCK, L - i * BLOCK)
                for j in range(i + 1):
                    if not self.block_mask[b, i, j]:
                        continue
                    if j < i:
                        tot += rows * BLOCK
                    else:
                        tot += rows * (rows + 1) // 2
        return tot

    def flops(self) -> int:
        """Algorithmic FLOPs: 2 * Hq * (D_qk + D_v) per visible pair."""
        return 2 * self.Hq * (self.D_qk + self.D_v) * self.visible_pairs()


def make_prefill_case(
    *,
    name: str,
    seed: int,
    seq_lens: Sequence[int],
    Hq: int,
    Hk: int,
    D_qk: int,
    D_rope: int,
    D_v: int,
    mask_density: Optional[float] = None,
    scale: Optional[float] = None,
) -> PrefillCase:
    """Draw a ragged prefill problem (token-major, sequences packed back to back).

    Draw order: q -> k -> v -> k_rope -> mask.  The block mask, when asked for,
    is uint8 [B, nb, nb] with nb = ceil(max_len / 64): each strictly-lower
    block is on with probability ``mask_density``, the diagonal and the first
    key block column are always on, and the upper triangle is off."""
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    B = seq_lens.shape[0]
    cu = np.zeros(B + 1, np.int32)
    cu[1:] = np.cumsum(seq_lens)
    T = int(cu[-1])
    ss = np.random.SeedSequence(seed)
    s_q, s_k, s_v, s_r, s_m = ss.spawn(5)
    D_nope = D_qk - D_rope
    q = to_bf16_bits(normal_f32(s_q, T * Hq * D_qk).reshape(T, Hq, D_qk))
    k = to_bf16_bits(normal_f32(s_k, T * Hk * D_nope).reshape(T, Hk, D_nope))
    v = to_bf16_bits(normal_f32(s_v, T * Hk * D_v).reshape(T, Hk, D_v))
    k_rope = None
    if D_rope:
        k_rope = to_bf16_bits(normal_f32(s_r, T * D_rope).reshape(T, 1, D_rope))
    block_mask = None
    if mask_density is not None:
        nb = (int(seq_lens.max()) + BLOCK - 1) // BLOCK
        g = np.random.Generator(np.random.PCG64(s_m))
        on = g.random((B, nb, nb)) < mask_density
        m = np.tril(on, -1)
        idx = np.arange(nb)
        m[:, idx, idx] = True
        m[:, :, 0] = True
        m = np.tril(m)
        block_mask = m.astype(np.uint8)
    if scale is None:
        scale = 1.0 / math.sqrt(D_qk)
    return PrefillCase(name=name, seq_lens=seq_lens, cu_seqlens=cu, Hq=Hq, Hk=Hk,
                       D_qk=D_qk, D_rope=D_rope, D_v=D_v, q=q, k=k, v=v, k_rope=k_rope,
                       block_mask=block_mask, scale=float(scale), meta={"seed": seed})


def _bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).float().numpy()


def make_prefill_fp8_case(
    *,
    name: str,
    seed: int,
    seq_lens: Sequence[int],
    Hq: int,
    Hk: int,
    D_rope: int = 64,
    mask_density: Optional[float] = None,
    scale: Optional[float] = None,
    blockwise: bool = False,
) -> PrefillCase:
    """The bf16 prefill problem of make_prefill_case (same seed, same draws,
    Dn = 128, Dv = 128), with the nope part of Q and all of K quantised to fp8
    e4m3fn with scale amax / 448 (the fp8 KV recipe): per tensor, or with
    ``blockwise`` per row of a head (a 1 x 128 block), giving float32 scale
    arrays [T, Hq] and [T, Hk] (an all-zero row gets scale 1).  The rope parts
    and V stay bf16.  scale defaults to 1/sqrt(128 + D_rope)."""
    base = make_prefill_case(name=name, seed=seed, seq_lens=seq_lens, Hq=Hq, Hk=Hk, D_qk=128 + D_rope,
                             D_rope=D_rope, D_v=128, mask_density=mask_density, scale=scale)
    qf = _bf16_bits_to_f32(base.q[:, :, :128])
    kf = _bf16_bits_to_f32(base.k)
    scales, codes = [], []
    for x in (qf, kf):
        if blockwise:
            amax = np.abs(x).max(axis=2) if x.size else np.ones(x.shape[:2], np.float32)
            sc = np.where(amax > 0, amax.astype(np.float32) / np.float32(E4M3FN_MAX), np.float32(1.0))
            sc = sc.astype(np.float32)
            codes.append(to_e4m3fn_bits(x, sc[..., None]))
        else:
            amax = float(np.abs(x).max()) if x.size else 1.0
            sc = float(np.float32(amax) / np.float32(E4M3FN_MAX)) if amax > 0 else 1.0
            codes.append(to_e4m3fn_bits(x, sc))
        scales.append(sc)
    base.q_rope = np.ascontiguousarray(base.q[:, :, 128:]) if D_rope else None
    base.q, base.k = codes
    base.q_scale, base.k_scale = scales
    base.dtype = "e4m3fn"
    return base


def make_prefill_rope_fp8_case(
    *,
    name: str,
    seed: int,
    seq_lens: Sequence[int],
    Hq: int,
    Hk: int,
    D_rope: int = 64,
    mask_density: Optional[float] = None,
    scale: Optional[float] = None,
) -> PrefillCase:
    """The bf16 MLA prefill problem of make_prefill_case (same seed, same
    draws, Dn = 128, Dv = 128) with the shared rope key quantised to fp8
    e4m3fn row by row: the scale of token t's rope row is amax over the row /
    448 (1 for an all-zero row), the codes those of the row over its scale.
    q, k and v stay bf16."""
    base = make_prefill_case(name=name, seed=seed, seq_lens=seq_lens, Hq=Hq, Hk=Hk, D_qk=128 + D_rope,
                             D_rope=D_rope, D_v=128, mask_density=mask_density, scale=scale)
    x = _bf16_bits_to_f32(base.k_rope)                                     # [T, 1, Dr]
    amax = np.abs(x).max(axis=(1, 2)) if x.size else np.ones(x.shape[0], np.float32)
    sc = np.where(amax > 0, amax.astype(np.float32) / np.float32(E4M3FN_MAX), np.float32(1.0)).astype(np.float32)
    base.k_rope = to_e4m3fn_bits(x, sc[:, None, None])
    base.k_rope_scale = sc
    base.rope_dtype = "e4m3fn"
    return base


def prefill_mla_bf16(seed: int = 1003, seq_lens=(512, 1024, 2048, 3000)) -> PrefillCase:
    """Ragged MLA prefill: 16 heads, Q 192 = 128 nope + 64 rope, K_rope shared
    [T, 1, 64], V / output 128, causal, scale 1/sqrt(192)."""
    return make_prefill_case(name="prefill_mla_bf16", seed=seed, seq_lens=seq_lens,
                             Hq=16, Hk=16, D_qk=192, D_rope=64, D_v=128)


def prefill_blocksparse_bf16(seed: int = 1005, P: int = 8192, B: int = 2) -> PrefillCase:
    """Block-sparse causal prefill: B=2, P=8192, Hq=32, Hk=8, D=128, 64x64 block
    mask with ~25% of the strictly-lower blocks on."""
    return make_prefill_case(name="prefill_blocksparse_bf16", seed=seed, seq_lens=[P] * B,
                             Hq=32, Hk=8, D_qk=128, D_rope=0, D_v=128, mask_density=0.25)


def prefill_mla_fp8(seed: int = 1009, seq_lens=(512, 1024, 2048, 3000)) -> PrefillCase:
    """The ragged MLA prefill shape (16 heads, Q 128 nope + 64 rope, shared
    K_rope, V / output 128, causal, scale 1/sqrt(192)) with q_nope and K in fp8
    e4m3fn, one scale each; q_rope, K_rope and V bf16."""
    return make_prefill_fp8_case(name="prefill_mla_fp8", seed=seed, seq_lens=seq_lens, Hq=16, Hk=16, D_rope=64)


def prefill_mla_fp8_blockwise(seed: int = 1010, seq_lens=(512, 1024, 2048, 3000)) -> PrefillCase:
    """prefill_mla_fp8 with one scale per row of a head (1 x 128 blocks of
    q_nope and K) instead of one per tensor."""
    return make_prefill_fp8_case(name="prefill_mla_fp8_blockwise", seed=seed, seq_lens=seq_lens, Hq=16, Hk=16,
                                 D_rope=64, blockwise=True)


def prefill_mla_rope_fp8(seed: int = 1012, seq_lens=(512, 1024, 2048, 3000)) -> PrefillCase:
    """The ragged MLA prefill shape (16 heads, Q 128 nope + 64 rope, V /
    output 128, causal, scale 1/sqrt(192)) with the shared rope key in fp8
    e4m3fn, one scale per rope row; q, k and v bf16."""
    return make_prefill_rope_fp8_case(name="prefill_mla_rope_fp8", seed=seed, seq_lens=seq_lens, Hq=16, Hk=16)


# ---------------------------------------------------------------------------
# Chunked prefill against a paged KV cache
# ---------------------------------------------------------------------------

@dataclass
class ChunkCase:
    name: str
    kv_lens: np.ndarray       # [B] int32: keys after the chunk is appended
    cu_seqlens_q: np.ndarray  # [B+1] int32: the chunks packed back to back
    Hq: int
    Hk: int
    D: int
    q: np.ndarray             # [T, Hq, D] bf16 bits
    k_new: np.ndarray         # [T, Hk, D] bf16 bits: the chunk's keys
    v_new: np.ndarray         # [T, Hk, D]
    k_pool: np.ndarray        # [NB, Hk, 64, D] bf16 bits: prefix rows filled, the rest NaN
    v_pool: np.ndarray
    block_table: np.ndarray   # [B, Nblk] int32 (-1 past ceil(kv_len / 64))
    scale: float
    kr_new: Optional[np.ndarray] = None    # MLA: [T, 1, Dr] bf16 bits, the chunk's rope keys
    kr_pool: Optional[np.ndarray] = None   # MLA: [NB, 1, 64, Dr] bf16 bits, rope cache on the same pages
    kv_dtype: str = "bf16"                 # 'e4m3fn': k_pool / v_pool hold fp8 codes (k_new / v_new stay bf16)
    k_scale: float = 1.0                   # fp8 pools: the value of code c is e4m3fn(c) * scale
    v_scale: float = 1.0
    meta: dict = field(default_factory=dict)

    @property
    def D_rope(self) -> int:
        return 0 if self.kr_pool is None else int(self.kr_pool.shape[3])

    @property
    def B(self) -> int:
        return int(self.kv_lens.shape[0])

    @property
    def T(self) -> int:
        return int(self.cu_seqlens_q[-1])

    @property
    def q_lens(self) -> np.ndarray:
        return np.diff(self.cu_seqlens_q).astype(np.int32)

    def visible_pairs(self) -> int:
        """(query, key) pairs the bottom-right aligned causal rule lets through."""
        n = 0
        for Lk, ql in zip(self.kv_lens.tolist(), self.q_lens.tolist()):
            off = Lk - ql
            # query i sees min(Lk, off + i + 1) keys (off >= 0 in every generated case)
            n += sum(min(Lk, off + i + 1) for i in range(ql))
        return n

    def flops(self) -> int:
        return 2 * self.Hq * (self.D + self.D_rope + self.D) * self.visible_pairs()


def make_chunk_case(
    *,
    name: str,
    seed: int,
    prefix_lens: Sequence[int],
    q_lens: Sequence[int],
    Hq: int,
    Hk: int,
    D: int = 128,
    D_rope: int = 0,
    spare_blocks: int = 2,
    scale: Optional[float] = None,
    kv_dtype: str = "bf16",
) -> ChunkCase:
    """Draw a chunked-prefill problem: sequence b already holds prefix_lens[b]
    keys in a paged bf16 cache and appends a chunk of q_lens[b] tokens.
    With kv_dtype 'e4m3fn' the K and V pools are an fp8 cache: the same draws,
    quantised with the per-tensor scale amax / 448, the amax taken over the
    pool's values and the chunk's new bf16 values together (so the append
    does not saturate); unused rows hold the NaN code.

    Draw order: block_table permutation -> q -> k_new -> v_new -> k_pool -> v_pool
    (-> kr_new -> kr_pool with a rope width D_rope: MLA, one rope head per token on
    the same pages; q then has D + D_rope columns).
    The pool has sum(ceil(kv_len / 64)) + spare_blocks blocks; the logical blocks
    (b, j) in row-major order take a seeded permutation of the pool ids.  Pool
    rows at or past each prefix (where the chunk will be appended), the rows past
    kv_len and the spare blocks are NaN.
    """
    ss = np.random.SeedSequence(seed)
    s_tab, s_q, s_kn, s_vn, s_k, s_v, s_rn, s_r = ss.spawn(8)
    prefix = np.asarray(prefix_lens, dtype=np.int32)
    ql = np.asarray(q_lens, dtype=np.int32)
    B = prefix.shape[0]
    kv_lens = (prefix + ql).astype(np.int32)
    need = _blocks_needed(kv_lens)
    nblk = max(1, int(need.max()) if B else 1)
    NB = int(need.sum()) + spare_blocks
    perm = np.random.Generator(np.random.PCG64(s_tab)).permutation(NB)
    block_table = np.full((B, nblk), -1, np.int32)
    k = 0
    for b in range(B):
        for j in range(int(need[b])):
            block_table[b, j] = perm[k]
            k += 1
    cu = np.zeros(B + 1, np.int32)
    cu[1:] = np.cumsum(ql)
    T = int(cu[-1])
    q = to_bf16_bits(normal_f32(s_q, T * Hq * (D + D_rope)).reshape(T, Hq, D + D_rope))
    k_new = to_bf16_bits(normal_f32(s_kn, T * Hk * D).reshape(T, Hk, D))
    v_new = to_bf16_bits(normal_f32(s_vn, T * Hk * D).reshape(T, Hk, D))
    keep = np.zeros((NB, BLOCK), bool)
    for b in range(B):
        for t in range(int(prefix[b])):
            keep[block_table[b, t // BLOCK], t % BLOCK] = True
    pools = []
    scales = [1.0, 1.0]
    for i, (s_x, heads, width) in enumerate(((s_k, Hk, D), (s_v, Hk, D), (s_r, 1, D_rope))):
        if width == 0:
            pools.append(None)
            continue
        xf = normal_f32(s_x, NB * heads * BLOCK * width).reshape(NB, heads, BLOCK, width)
        if kv_dtype == "e4m3fn" and i < 2:
            new = _bf16_bits_to_f32(k_new if i == 0 else v_new)
            amax = max(float(np.abs(xf).max()) if xf.size else 0.0, float(np.abs(new).max()) if new.size else 0.0)
            sc = float(np.float32(amax) / np.float32(E4M3FN_MAX)) if amax > 0 else 1.0
            x = to_e4m3fn_bits(xf, sc)
            x.transpose(0, 2, 1, 3)[~keep] = E4M3FN_NAN
            scales[i] = sc
        elif kv_dtype in ("bf16", "e4m3fn"):
            x = to_bf16_bits(xf)
            x.transpose(0, 2, 1, 3)[~keep] = BF16_NAN
        else:
            raise ValueError(kv_dtype)
        pools.append(x)
    kr_new = to_bf16_bits(normal_f32(s_rn, T * D_rope).reshape(T, 1, D_rope)) if D_rope else None
    if scale is None:
        scale = 1.0 / math.sqrt(D + D_rope)
    return ChunkCase(name=name, kv_lens=kv_lens, cu_seqlens_q=cu, Hq=Hq, Hk=Hk, D=D, q=q, k_new=k_new,
                     v_new=v_new, k_pool=pools[0], v_pool=pools[1], block_table=block_table,
                     scale=float(scale), kr_new=kr_new, kr_pool=pools[2], kv_dtype=kv_dtype,
                     k_scale=scales[0], v_scale=scales[1], meta={"seed": seed, "prefix_lens": prefix})


def prefill_chunk_bf16(seed: int = 1006, B: int = 8, prefix_range=(1024, 6144), q_len: int = 512) -> ChunkCase:
    """Chunked prefill: B=8 sequences with cached prefixes ~ U{1024..6144}
    appending 512-token chunks; Hq=32, Hk=8, D=128, bf16, paged 64-row cache."""
    lo, hi = prefix_range
    prefix = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed).spawn(1)[0])).integers(lo, hi + 1, size=B)
    return make_chunk_case(name="prefill_chunk_bf16", seed=seed + 1, prefix_lens=prefix.tolist(),
                           q_lens=[q_len] * B, Hq=32, Hk=8, D=128)


def prefill_chunk_mla_bf16(seed: int = 1008, B: int = 4, prefix_range=(1024, 4096), q_len: int = 512) -> ChunkCase:
    """MLA chunked prefill: 4 sequences with cached prefixes ~ U{1024..4096}
    appending 512-token chunks; 16 heads, Q 192 = 128 + 64 rope, the rope keys
    in a one-head paged rope cache, V / output 128, bf16."""
    lo, hi = prefix_range
    prefix = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed).spawn(1)[0])).integers(lo, hi + 1, size=B)
    return make_chunk_case(name="prefill_chunk_mla_bf16", seed=seed + 1, prefix_lens=prefix.tolist(),
                           q_lens=[q_len] * B, Hq=16, Hk=16, D=128, D_rope=64)


def prefill_chunk_long_mla_bf16(seed: int = 1011, prefix: int = 15872, q_len: int = 512) -> ChunkCase:
    """Long-context MLA chunked prefill: one sequence with a 15872-token cached
    prefix appending a 512-token chunk (16384 keys); 16 heads, Q 192 = 128 + 64
    rope, the rope keys in the paged rope cache, V / output 128, bf16."""
    return make_chunk_case(name="prefill_chunk_long_mla_bf16", seed=seed, prefix_lens=[prefix], q_lens=[q_len],
                           Hq=16, Hk=16, D=128, D_rope=64)


def prefill_chunk_fp8kv(seed: int = 1006, B: int = 8, prefix_range=(1024, 6144), q_len: int = 512) -> ChunkCase:
    """Chunked prefill over an fp8 e4m3fn KV cache: the shapes and draws of
    prefill_chunk_bf16 (B=8, cached prefixes ~ U{1024..6144}, 512-token chunks,
    Hq=32, Hk=8, D=128, bf16 queries), the K and V pools quantised with the
    per-tensor scale amax / 448 as in the fp8 decode workload."""
    lo, hi = prefix_range
    prefix = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed).spawn(1)[0])).integers(lo, hi + 1, size=B)
    return make_chunk_case(name="prefill_chunk_fp8kv", seed=seed + 1, prefix_lens=prefix.tolist(),
                           q_lens=[q_len] * B, Hq=32, Hk=8, D=128, kv_dtype="e4m3fn")


def decode_multitoken(q_len: int, seed: int = 1013, B: int = 64, len_range=(1024, 4096), Hq: int = 32,
                      Hk: int = 8, D_rope: int = 0) -> ChunkCase:
    """Multi-token decode: every sequence holds kv_len ~ U{len_range} keys in a
    paged cache (the paged-decode workload's shape: B=64, Hq=32, Hk=8, D=128), the last q_len of
    them new tokens whose queries attend causally (bottom-right aligned).  With
    D_rope = 64 it is the MLA form (per-head K plus one shared rope row per
    token from the rope cache)."""
    ss = np.random.SeedSequence(seed)
    kv = np.random.Generator(np.random.PCG64(ss.spawn(1)[0])).integers(len_range[0], len_range[1] + 1, size=B)
    name = f"decode_mt{q_len}" + ("_mla" if D_rope else "") + "_bf16"
    c = make_chunk_case(name=name, seed=seed + 1, prefix_lens=(kv - q_len).tolist(), q_lens=[q_len] * B, Hq=Hq,
                        Hk=Hk, D_rope=D_rope)
    c.meta["seed"] = seed
    return c


def kv_read_bytes(case: "ChunkCase") -> int:
    """Bytes of cache rows a decode over the case's keys must read: K and V of
    every key and KV head (bf16), plus the shared rope row of every key."""
    n = int(case.kv_lens.astype(np.int64).sum())
    esz = 1 if case.kv_dtype == "e4m3fn" else 2
    return n * case.Hk * case.D * 2 * esz + n * case.D_rope * 2


CONFIGS = {
    "decode_tiny_f32": decode_tiny_fp32,
    "decode_gqa_bf16": decode_gqa_bf16,
    "prefill_mla_bf16": prefill_mla_bf16,
    "decode_long_fp8": decode_long_fp8,
    "prefill_blocksparse_bf16": prefill_blocksparse_bf16,
    "prefill_chunk_bf16": prefill_chunk_bf16,
    "prefill_chunk_mla_bf16": prefill_chunk_mla_bf16,
    "prefill_mla_fp8": prefill_mla_fp8,
    "prefill_mla_fp8_blockwise": prefill_mla_fp8_blockwise,
    "prefill_chunk_long_mla_bf16": prefill_chunk_long_mla_bf16,
    "prefill_chunk_fp8kv": prefill_chunk_fp8kv,
    "prefill_mla_rope_fp8": prefill_mla_rope_fp8,
    "decode_mt1_bf16": lambda: decode_multitoken(1),
    "decode_mt2_bf16": lambda: decode_multitoken(2),
    "decode_mt4_bf16": lambda: decode_multitoken(4),
    "decode_mt2_mla_bf16": lambda: decode_multitoken(2, Hq=16, Hk=16, D_rope=64),
}
