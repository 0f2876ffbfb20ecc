"""CPU fp64 oracle for paged GQA decode and ragged (MLA) prefill attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this module; only the tests, the smoke check and the benchmark's CPU-baseline
leg do.  It shares no code with the device library: it reads the storage bits
produced by the input generator and widens them with its own code.

What it computes is the plain definition of attention, evaluated in float64
over the logically gathered sequence:

  out[h] = sum_t softmax_t(scale * <q[h], K[t]>) * V[t]
  lse[h] = log(sum_t exp(scale * <q[h], K[t]>))           (natural log)

Paging, splitting, tiling and block skipping in the device path are only
faster ways to the same value, so none of them appear here.

Sources (the pages this follows):
  * FlashMLA "Tensor Shapes Reference", section 1 (flash_mla_with_kvcache):
    q [B, Hq, 1, D], a paged K/V cache of 64-row blocks, block_table [B, Nblk]
    mapping a sequence's block index to a physical cache block, seq_lens [B];
    the last block may be partly filled and the unused slots are ignored by
    seq_lens.  Same page, "Grouped-Query Attention" diagram: q heads 2g and
    2g+1 of an 8:4 model read KV head g, i.e. kv head = h // (Hq / Hk).  Same
    page, "Prefill to Cache Mapping": tokens 64j .. 64j+63 live in
    block_table[b, j].
  * Modular "flare_mla_prefill": ragged Q [tokens, heads, 192], K and V
    [tokens, heads, 128], K_rope [tokens, 1, 64]; the 64 missing elements of
    each K head are the shared rope key broadcast to all heads; the output has
    the reduced (V) width; per-sequence valid lengths.
  * MATE msa_interface: fp8 KV is torch.float8_e4m3fn with per-tensor k_scale
    and v_scale (the _run_sparse_fwd_kernel argument list); cu_seqlens is
    [0, cumsum(lengths)] (_make_cu_seqlens); with equal query and key lengths
    the causal offset kv_len - q_len is 0 (_normalize_qo_offset), so query i
    sees keys j <= i.
  * FlashMLA "Tensor Shapes Reference", section 3 (flash_mla_prefill): an
    optional block-sparse pattern, block-aligned to 64.

  * FlashMLA "Tensor Shapes Reference", section 4 (mha_fwd_kvcache) and its
    "Prefill to Cache Mapping" diagram: a prefill writes its keys and values
    into the paged cache, tokens 64j .. 64j+63 of a sequence going to
    block_table[b, j].  MATE msa_interface: without an explicit offset the
    query chunk is aligned to the end of the keys (_normalize_qo_offset gives
    kv_len - q_len), and a causal query i then uses keys up to i + offset
    (_resolve_seqused_k).

Readings where the pages are silent (each also listed in the design notes):
  * the KV cache is one shared physical pool [NB, Hk, 64, D]; block ids are
    global; table entries past ceil(L/64) are padding and never read;
  * the decode query is the newest token and sees all L keys;
  * block-sparse prefill: key j is visible to query i iff j <= i and
    mask[b, i // 64, j // 64] != 0 (a diagonal block that is off hides it);
  * a row with no visible key has out = 0 and lse = -inf;
  * fp8 values are e4m3fn(byte) * scale, with the pool's per-tensor scale;
  * fp8 prefill: q_nope and K carry one scale per tensor, or one per row of
    a head (a 1 x 128 block: q_scale [T, Hq], k_scale [T, Hk]); the page leaves
    the layout of q_scale and k_scales open and these are the two plainest
    ones; the rope parts and V are bf16 and unscaled;
  * chunked prefill: a sequence holds kv_len keys in the paged cache, the last
    q_len of which are the chunk's own tokens (appended at logical positions
    kv_len - q_len + i); query i sees key j iff j <= kv_len - q_len + i.
  * quantised rope key: the shared rope key rows are e4m3fn codes with one
    fp32 scale per row (token), the value of a code being e4m3fn(code) times
    its row's scale; the query, the per-head keys and V stay bf16.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

BLOCK = 64


# --------------------------------------------------------------------------
# Storage formats -> float64
# --------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 is the top half of an IEEE binary32: widen by shifting the 16 bits up."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def e4m3fn_table() -> np.ndarray:
    """Value of each of the 256 OCP fp8 E4M3FN codes (1 sign, 4 exponent bits with
    bias 7, 3 mantissa bits; no infinities; S.1111.111 is NaN; exponent field 0
    holds the subnormals m * 2**-9)."""
    tab = np.empty(256, np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            tab[code] = math.nan
        elif e == 0:
            tab[code] = sign * m * 2.0 ** -9
        else:
            tab[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return tab


_E4M3FN = e4m3fn_table()


def quantize_e4m3fn(x: np.ndarray, scale: float) -> np.ndarray:
    """Codes of x / scale in OCP fp8 E4M3FN (the writer's side of a per-tensor
    scaled fp8 cache: the stored code c stands for e4m3fn(c) * scale).

    The quotient is taken in float32 (x is float32; IEEE division, correctly
    rounded).  Its code is the one whose value is nearest, ties going to the
    code with an even last mantissa bit (round to nearest even); magnitudes
    past the largest finite value 448 saturate to it (the format has no
    infinities); the sign of zero is kept; NaN gives the NaN code with its
    sign.  Returns uint8 codes."""
    with np.errstate(over="ignore"):          # a quotient past float32 range saturates below
        y = np.asarray(x, dtype=np.float32) / np.float32(scale)
    a = np.abs(y).astype(np.float64)
    pos = _E4M3FN[:0x7F]                       # values of codes 0x00 .. 0x7E, ascending
    hi = np.clip(np.searchsorted(pos, a, side="left"), 0, 0x7E)   # first code with value >= a
    lo = np.clip(hi - 1, 0, 0x7E)
    d_hi = pos[hi] - a
    d_lo = a - pos[lo]
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (lo % 2 == 0))
    code = np.where(pick_lo, lo, hi)
    code = np.where(a >= pos[0x7E], 0x7E, code)                     # saturate at 448
    code = code.astype(np.uint8)
    code |= np.where(np.signbit(y), np.uint8(0x80), np.uint8(0))
    code = np.where(np.isnan(y), np.where(np.signbit(y), np.uint8(0xFF), np.uint8(0x7F)), code)
    return code.astype(np.uint8)


def e4m3fn_to_f64(bits: np.ndarray) -> np.ndarray:
    return _E4M3FN[np.asarray(bits, dtype=np.uint8)]


def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Storage bits (as produced by the input generator) -> float64 values."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_to_f64(x)
    if dtype == "e4m3fn":
        return e4m3fn_to_f64(x)
    if dtype == "f64":
        return np.asarray(x, dtype=np.float64)
    raise ValueError(f"unknown dtype tag {dtype!r}")


# --------------------------------------------------------------------------
# Paged decode
# --------------------------------------------------------------------------

def gather_kv_rows(pool: np.ndarray, block_table: np.ndarray, b: int, g: int, L: int) -> np.ndarray:
    """Logical rows 0..L-1 of KV head g of sequence b, in storage format (exact).

    Row t is row t % 64 of physical block block_table[b, t // 64]; only the
    first ceil(L / 64) entries of the table row are read."""
    nb = (L + BLOCK - 1) // BLOCK
    phys = np.asarray(block_table[b, :nb], dtype=np.int64)
    rows = pool[phys, g]                      # [nb, 64, D]
    return rows.reshape(nb * BLOCK, pool.shape[-1])[:L]


def _softmax_attend(s: np.ndarray, V: np.ndarray):
    """s: [..., L] scores (with -inf for hidden keys); V: [L, Dv].
    Returns (out [..., Dv], lse [...]).  No visible key -> out 0, lse -inf."""
    m = s.max(axis=-1, initial=-np.inf)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    w = np.exp(s - m_safe[..., None])          # exp(-inf) = 0 for hidden keys
    l = w.sum(axis=-1)
    num = w @ V
    with np.errstate(invalid="ignore", divide="ignore"):
        out = np.where((l > 0)[..., None], num / np.where(l > 0, l, 1.0)[..., None], 0.0)
        lse = np.where(l > 0, m_safe + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return out, lse


def paged_decode(
    q: np.ndarray,
    k_pool: np.ndarray,
    v_pool: np.ndarray,
    block_table: np.ndarray,
    seq_lens: np.ndarray,
    scale: float,
    *,
    q_dtype: str = "f64",
    kv_dtype: str = "f64",
    k_scale: float = 1.0,
    v_scale: float = 1.0,
    batches: Optional[Sequence[int]] = None,
):
    """Single-token decode over a paged KV cache with grouped-query heads.

    q [B, Hq, D]; k_pool, v_pool [NB, Hk, 64, D]; block_table [B, Nblk] int;
    seq_lens [B].  Inputs are storage bits tagged by q_dtype / kv_dtype (or
    float64 with tag 'f64').  Returns (out [nb, Hq, D], lse [nb, Hq]) in
    float64 for the sequences in ``batches`` (default: all, in order)."""
    B, Hq, D = q.shape
    Hk = k_pool.shape[1]
    if Hq % Hk:
        raise ValueError("Hq must be a multiple of Hk")
    r = Hq // Hk
    if batches is None:
        batches = range(B)
    batches = list(batches)
    out = np.zeros((len(batches), Hq, D), np.float64)
    lse = np.full((len(batches), Hq), -np.inf, np.float64)
    for i, b in enumerate(batches):
        L = int(seq_lens[b])
        qb = widen(q[b], q_dtype)                           # [Hq, D]
        for g in range(Hk):
            K = widen(gather_kv_rows(k_pool, block_table, b, g, L), kv_dtype) * k_scale
            V = widen(gather_kv_rows(v_pool, block_table, b, g, L), kv_dtype) * v_scale
            heads = slice(g * r, (g + 1) * r)               # kv head g serves q heads g*r .. g*r+r-1
            s = scale * (qb[heads] @ K.T)                   # [r, L]
            o, ls = _softmax_attend(s, V)
            out[i, heads] = o
            lse[i, heads] = ls
    return out, lse


# --------------------------------------------------------------------------
# Ragged prefill (causal, optional MLA rope key, optional 64x64 block mask)
# --------------------------------------------------------------------------

def ragged_prefill(
    q: np.ndarray,
    k: np.ndarray,
    v: np.ndarray,
    cu_seqlens: np.ndarray,
    scale: float,
    *,
    k_rope: Optional[np.ndarray] = None,
    block_mask: Optional[np.ndarray] = None,
    dtype: str = "f64",
    rows: Optional[Sequence[int]] = None,
    row_chunk: int = 256,
):
    """Causal attention over sequences packed back to back (token-major).

    q [T, Hq, Dn + Dr]; k [T, Hk, Dn]; v [T, Hk, Dv]; k_rope [T, 1, Dr] or None
    (then Dr = 0); cu_seqlens [B + 1].  Query head h reads KV head h // (Hq/Hk).
    The score of query i and key j of one sequence is
        scale * (q[i, h, :Dn] . k[j, g] + q[i, h, Dn:] . k_rope[j, 0])
    and key j is visible iff j <= i and (no mask or mask[b, i//64, j//64]).

    ``rows``: optional global token indices to evaluate (default all), so that a
    sample of a large problem can be checked row by row.
    Returns (out [n, Hq, Dv], lse [n, Hq]) in float64."""
    Q = widen(q, dtype)
    K = widen(k, dtype)
    V = widen(v, dtype)
    KR = widen(k_rope, dtype) if k_rope is not None else None
    T, Hq, Dqk = Q.shape
    Hk, Dn = K.shape[1], K.shape[2]
    Dr = 0 if KR is None else KR.shape[2]
    if Dn + Dr != Dqk:
        raise ValueError("query width must equal K width plus rope width")
    if Hq % Hk:
        raise ValueError("Hq must be a multiple of Hk")
    r = Hq // Hk
    Dv = V.shape[2]
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    B = cu.shape[0] - 1
    if rows is None:
        rows = np.arange(T)
    rows = np.asarray(rows, dtype=np.int64)
    out = np.zeros((rows.shape[0], Hq, Dv), np.float64)
    lse = np.full((rows.shape[0], Hq), -np.inf, np.float64)
    seq_of_row = np.searchsorted(cu, rows, side="right") - 1
    for b in range(B):
        c0, c1 = int(cu[b]), int(cu[b + 1])
        sel = np.nonzero(seq_of_row == b)[0]
        if sel.size == 0 or c1 == c0:
            continue
        for s0 in range(0, sel.size, row_chunk):
            idx = sel[s0:s0 + row_chunk]
            gi = rows[idx]                    # global token ids of these queries
            i = gi - c0                       # local query positions
            n = idx.size
            # Keys past the last query of the chunk are causally hidden from
            # every row of it, so only keys 0 .. max(i) are scored.
            nk = int(i.max()) + 1
            j = np.arange(nk)
            vis = j[None, :] <= i[:, None]    # causal: key j visible to query i iff j <= i
            if block_mask is not None:
                vis &= block_mask[b][(i // BLOCK)[:, None], (j // BLOCK)[None, :]] != 0
            for g in range(Hk):
                heads = slice(g * r, (g + 1) * r)
                Qc = Q[gi, heads, :].reshape(n * r, Dqk)    # the r query heads of KV head g, row-major
                s = Qc[:, :Dn] @ K[c0:c0 + nk, g, :].T      # [n * r, nk]
                if KR is not None:
                    s = s + Qc[:, Dn:] @ KR[c0:c0 + nk, 0, :].T
                s = scale * s.reshape(n, r, nk)
                s = np.where(vis[:, None, :], s, -np.inf)
                o, ls = _softmax_attend(s, V[c0:c0 + nk, g, :])
                out[idx, heads] = o
                lse[idx, heads] = ls
    return out, lse


def cu_seqlens_from_lengths(lengths: Sequence[int]) -> np.ndarray:
    """[0, cumsum(lengths)] as int32 (length B + 1)."""
    lens = np.asarray(lengths, dtype=np.int64)
    cu = np.zeros(lens.shape[0] + 1, np.int64)
    cu[1:] = np.cumsum(lens)
    return cu.astype(np.int32)


# --------------------------------------------------------------------------
# Chunked prefill against a paged KV cache
# --------------------------------------------------------------------------

def append_kv(
    k_new: np.ndarray,
    v_new: np.ndarray,
    k_pool: np.ndarray,
    v_pool: np.ndarray,
    block_table: np.ndarray,
    cu_seqlens_q: np.ndarray,
    kv_lens: np.ndarray,
    *,
    kr_new: Optional[np.ndarray] = None,
    kr_pool: Optional[np.ndarray] = None,
    kv_dtype: str = "bf16",
    k_scale: float = 1.0,
    v_scale: float = 1.0,
):
    """Write a chunk's keys and values into the paged cache (storage bits, exact).

    k_new, v_new [T, Hk, D] hold the chunk tokens of all sequences back to back
    (cu_seqlens_q); sequence b's chunk is the last q_len_b = cu[b+1] - cu[b] of
    its kv_lens[b] keys, so its token i goes to logical position
    p = kv_lens[b] - q_len_b + i: row p % 64 of pool block block_table[b, p // 64]
    (FlashMLA tensor-shape reference, section 4, "Prefill to Cache Mapping").
    With an MLA rope cache, kr_new [T, 1, Dr] goes to kr_pool [NB, 1, 64, Dr]
    by the same rule (flare_mla_prefill, overload A: the rope keys live in a
    paged cache too).  Returns new pools ((k, v) or (k, v, kr)); the inputs
    are not modified.

    With kv_dtype "e4m3fn" the pools hold fp8 codes with per-tensor scales
    (the fp8 KV cache of decode): the chunk's bf16 keys and values are
    written as quantize_e4m3fn(value, k_scale) and (value, v_scale); the
    rope cache stays bf16."""
    if kv_dtype == "e4m3fn":
        k_new = quantize_e4m3fn(bf16_to_f64(k_new).astype(np.float32), k_scale)
        v_new = quantize_e4m3fn(bf16_to_f64(v_new).astype(np.float32), v_scale)
    elif kv_dtype != "bf16":
        raise ValueError(f"unknown kv dtype {kv_dtype!r}")
    kp = np.array(k_pool, copy=True)
    vp = np.array(v_pool, copy=True)
    rp = np.array(kr_pool, copy=True) if kr_pool is not None else None
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    for b in range(cu.shape[0] - 1):
        ql = int(cu[b + 1] - cu[b])
        first = int(kv_lens[b]) - ql
        for i in range(ql):
            p = first + i
            if p < 0:
                continue
            blk = int(block_table[b, p // BLOCK])
            kp[blk, :, p % BLOCK] = k_new[cu[b] + i]
            vp[blk, :, p % BLOCK] = v_new[cu[b] + i]
            if rp is not None:
                rp[blk, :, p % BLOCK] = kr_new[cu[b] + i]
    return (kp, vp) if rp is None else (kp, vp, rp)


def chunk_prefill(
    q: np.ndarray,
    k_pool: np.ndarray,
    v_pool: np.ndarray,
    block_table: np.ndarray,
    cu_seqlens_q: np.ndarray,
    kv_lens: np.ndarray,
    scale: float,
    *,
    dtype: str = "f64",
    rows: Optional[Sequence[int]] = None,
    row_chunk: int = 256,
    kr_pool: Optional[np.ndarray] = None,
    kv_dtype: Optional[str] = None,
    k_scale: float = 1.0,
    v_scale: float = 1.0,
):
    """Causal attention of a chunk of new queries to a paged KV cache.

    q [T, Hq, D] (chunks packed back to back, cu_seqlens_q [B + 1]); k_pool,
    v_pool [NB, Hk, 64, D]; block_table [B, Nblk]; kv_lens [B] counts every
    key of sequence b, the chunk's own tokens included.  With q_len_b =
    cu[b+1] - cu[b] and offset o_b = kv_lens[b] - q_len_b (the chunk aligned to
    the end of the keys), query i sees logical key j iff j < kv_lens[b] and
    j <= o_b + i.  Keys are gathered from the pool exactly as in decode.
    With kr_pool [NB, 1, 64, Dr] (MLA), q is [T, Hq, Dn + Dr] and the score of key
    j adds q[i, h, Dn:] . kr[j], the rope key of token j from the same pages,
    shared by every head (flare_mla_prefill: the K head lacks the rope part,
    which comes from the rope cache for all heads).
    ``rows``: optional global query indices to evaluate (default all).
    ``kv_dtype``: storage of the K/V pools when it differs from ``dtype``;
    "e4m3fn" pools hold fp8 codes whose values are e4m3fn(code) * k_scale
    (keys) and * v_scale (values), as for decode; the rope cache has ``dtype``.
    Returns (out [n, Hq, D], lse [n, Hq]) in float64."""
    Q = widen(q, dtype)
    kvd = dtype if kv_dtype is None else kv_dtype
    T, Hq, Dqk = Q.shape
    Hk, Dn = k_pool.shape[1], k_pool.shape[3]
    Dr = 0 if kr_pool is None else kr_pool.shape[3]
    if Dn + Dr != Dqk:
        raise ValueError("query width must equal K width plus rope width")
    if Hq % Hk:
        raise ValueError("Hq must be a multiple of Hk")
    r = Hq // Hk
    Dv = v_pool.shape[3]
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    B = cu.shape[0] - 1
    if rows is None:
        rows = np.arange(T)
    rows = np.asarray(rows, dtype=np.int64)
    out = np.zeros((rows.shape[0], Hq, Dv), np.float64)
    lse = np.full((rows.shape[0], Hq), -np.inf, np.float64)
    seq_of_row = np.searchsorted(cu, rows, side="right") - 1
    for b in range(B):
        sel = np.nonzero(seq_of_row == b)[0]
        Lk = int(kv_lens[b])
        if sel.size == 0 or Lk == 0:
            continue
        off = Lk - int(cu[b + 1] - cu[b])
        j = np.arange(Lk)
        KR = widen(gather_kv_rows(kr_pool, block_table, b, 0, Lk), dtype) if Dr else None
        for g in range(Hk):
            K = widen(gather_kv_rows(k_pool, block_table, b, g, Lk), kvd) * float(k_scale)
            V = widen(gather_kv_rows(v_pool, block_table, b, g, Lk), kvd) * float(v_scale)
            heads = slice(g * r, (g + 1) * r)
            for s0 in range(0, sel.size, row_chunk):
                idx = sel[s0:s0 + row_chunk]
                n = idx.size
                i = rows[idx] - cu[b]                      # local query index in the chunk
                # keys past off + max(i) are hidden from every row of the chunk
                nk = max(0, min(Lk, off + int(i.max()) + 1))
                vis = j[None, :nk] <= (off + i)[:, None]   # bottom-right aligned causal bound
                Qc = Q[rows[idx], heads, :].reshape(n * r, Dqk)
                s = Qc[:, :Dn] @ K[:nk].T                  # [n * r, nk]
                if Dr:
                    s = s + Qc[:, Dn:] @ KR[:nk].T
                s = scale * s.reshape(n, r, nk)
                s = np.where(vis[:, None, :], s, -np.inf)
                o, ls = _softmax_attend(s, V[:nk])
                out[idx, heads] = o
                lse[idx, heads] = ls
    return out, lse


# --------------------------------------------------------------------------
# CSR page input
# --------------------------------------------------------------------------

def block_table_from_csr(kv_indices: np.ndarray, kv_page_indptr: np.ndarray, max_blocks: int) -> np.ndarray:
    """Padded block table [B, max_blocks] from the flat page list of MATE
    msa_interface (_build_page_table_from_flat_kv_indices): the pages of
    sequence b are kv_indices[indptr[b] : indptr[b + 1]], in order; the rest of
    each row is padding (-1).  Pages past max_blocks are not represented."""
    ip = np.asarray(kv_page_indptr, dtype=np.int64)
    B = ip.shape[0] - 1
    table = np.full((B, max_blocks), -1, np.int32)
    for b in range(B):
        pages = np.asarray(kv_indices[ip[b]:ip[b + 1]], dtype=np.int32)[:max_blocks]
        table[b, :pages.shape[0]] = pages
    return table


# --------------------------------------------------------------------------
# fp8 MLA prefill (per-tensor scales)
# --------------------------------------------------------------------------

def ragged_prefill_fp8(
    q_nope: np.ndarray,
    q_rope: Optional[np.ndarray],
    k: np.ndarray,
    v: np.ndarray,
    k_rope: Optional[np.ndarray],
    cu_seqlens: np.ndarray,
    scale: float,
    q_scale,
    k_scale,
    *,
    block_mask: Optional[np.ndarray] = None,
    rows: Optional[Sequence[int]] = None,
):
    """Ragged causal prefill with the per-head (nope) parts of Q and K in fp8
    (Modular flare_mla_prefill, the overload taking q_nope, q_rope, q_scale and
    k_scales): q_nope [T, Hq, Dn] and k [T, Hk, Dn] hold e4m3fn codes;
    q_rope [T, Hq, Dr], k_rope [T, 1, Dr] and v [T, Hk, Dv] are bf16 (q_rope and
    k_rope both None for a model without the rope part).

    Scales: q_scale is one float for the whole tensor or an array [T, Hq] with
    one scale per row of a head (a 1 x Dn block); k_scale likewise, a float or
    [T, Hk].  The value of a code is e4m3fn(code) times the scale of its block,
    the query is those values followed by q_rope, and the rest is
    ragged_prefill on them:
        score = scale * (q_scale[i,h] * k_scale[j,g] * (codes of q_nope[i,h] . codes of k[j,g])
                         + q_rope[i,h] . k_rope[j])
    Returns (out [n, Hq, Dv], lse [n, Hq]) in float64."""
    if (q_rope is None) != (k_rope is None):
        raise ValueError("q_rope and k_rope go together")
    qs = np.asarray(q_scale, dtype=np.float64)
    ks = np.asarray(k_scale, dtype=np.float64)
    q = widen(q_nope, "e4m3fn") * (qs[..., None] if qs.ndim else qs)
    if q_rope is not None:
        q = np.concatenate([q, widen(q_rope, "bf16")], axis=2)
    kk = widen(k, "e4m3fn") * (ks[..., None] if ks.ndim else ks)
    kr = None if k_rope is None else widen(k_rope, "bf16")
    return ragged_prefill(q, kk, widen(v, "bf16"), cu_seqlens, scale, k_rope=kr, block_mask=block_mask,
                          dtype="f64", rows=rows)


# --------------------------------------------------------------------------
# MLA prefill with a quantised shared rope key
# --------------------------------------------------------------------------

def ragged_prefill_rope_fp8(
    q: np.ndarray,
    k: np.ndarray,
    v: np.ndarray,
    k_rope: np.ndarray,
    k_rope_scale,
    cu_seqlens: np.ndarray,
    scale: float,
    *,
    block_mask: Optional[np.ndarray] = None,
    rows: Optional[Sequence[int]] = None,
):
    """Ragged causal MLA prefill whose shared rope key is quantised (Modular
    flare_mla_prefill, the overload that takes k_rope together with
    k_rope_scales): q [T, Hq, Dn + Dr], k [T, Hk, Dn] and v [T, Hk, Dv] are bf16;
    k_rope [T, 1, Dr] holds e4m3fn codes and k_rope_scale [T] one float32
    scale per rope row.  The value of a rope code is e4m3fn(code) times its
    row's scale (a per-tensor scale is the case of equal entries), and the
    rest is ragged_prefill on those values:
        score = scale * (q[i,h,:Dn] . k[j,g] + k_rope_scale[j] * (q[i,h,Dn:] . codes of k_rope[j]))
    Returns (out [n, Hq, Dv], lse [n, Hq]) in float64."""
    ks = np.asarray(k_rope_scale, dtype=np.float64)
    if ks.shape != (k_rope.shape[0],):
        raise ValueError("k_rope_scale holds one scale per rope row")
    kr = widen(k_rope, "e4m3fn") * ks[:, None, None]
    return ragged_prefill(widen(q, "bf16"), widen(k, "bf16"), widen(v, "bf16"), cu_seqlens, scale, k_rope=kr,
                          block_mask=block_mask, dtype="f64", rows=rows)
