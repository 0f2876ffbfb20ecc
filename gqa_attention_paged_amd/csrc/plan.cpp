// Host-only planning and validation (no device calls).
//
// Decode plan: the FlashMLA tensor-shape reference describes get_mla_metadata
// as shape/stride validation that materialises nothing, and lists the shape
// mistakes a caller can make (Hq not a multiple of Hk, sequences longer than
// Nblk*64, a block size other than 64, non-contiguous inner dims, q and cache
// of different dtypes).  MATE's planner sizes its schedule from capacities so
// that execution never reads lengths on the host; the split count here is
// likewise a function of the descriptor only.
#include <algorithm>
#include <climits>
#include <cstring>
#include <string>

#include "status.hpp"

namespace gqap {

std::string& last_error_slot() {
  static thread_local std::string msg;
  return msg;
}

static bool elem_size(int32_t dt, int* out) {
  switch (dt) {
    case GQAP_F32: *out = 4; return true;
    case GQAP_BF16: *out = 2; return true;
    case GQAP_FP8_E4M3FN: *out = 1; return true;
    case GQAP_F16: *out = 2; return true;
    default: return false;
  }
}

// A stride in elements keeps 16-byte vector accesses aligned.
static bool aligned16(int64_t stride_elems, int esz) { return (stride_elems * esz) % 16 == 0; }

static gqap_status check_decode_desc(const gqap_decode_desc_t& d, int* q_esz, int* kv_esz) {
  if (d.batch < 0 || d.batch > 65535)
    return fail(GQAP_ERR_INVALID_ARGUMENT, "batch must be in [0, 65535] (got %d)", d.batch);
  if (d.num_q_heads <= 0 || d.num_kv_heads <= 0)
    return fail(GQAP_ERR_INVALID_ARGUMENT, "head counts must be positive (Hq=%d, Hk=%d)", d.num_q_heads,
                d.num_kv_heads);
  if (d.num_q_heads % d.num_kv_heads)
    return fail(GQAP_ERR_INVALID_ARGUMENT, "Hq (%d) must be a multiple of Hk (%d)", d.num_q_heads, d.num_kv_heads);
  if (d.block_size != kBlock)
    return fail(GQAP_ERR_UNSUPPORTED, "block_size must be %d (got %d)", kBlock, d.block_size);
  if (d.head_dim != 64 && d.head_dim != 128)
    return fail(GQAP_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", d.head_dim);
  if (!elem_size(d.q_dtype, q_esz)) return fail(GQAP_ERR_DTYPE, "unknown q_dtype %d", d.q_dtype);
  if (!elem_size(d.kv_dtype, kv_esz)) return fail(GQAP_ERR_DTYPE, "unknown kv_dtype %d", d.kv_dtype);
  if (d.q_dtype == GQAP_F16 || d.kv_dtype == GQAP_F16)
    return fail(GQAP_ERR_UNSUPPORTED, "fp16 is not implemented");
  const bool ok_pair = (d.q_dtype == GQAP_F32 && d.kv_dtype == GQAP_F32) ||
                       (d.q_dtype == GQAP_BF16 && d.kv_dtype == GQAP_BF16) ||
                       (d.q_dtype == GQAP_BF16 && d.kv_dtype == GQAP_FP8_E4M3FN);
  if (!ok_pair)
    return fail(GQAP_ERR_DTYPE, "dtype pair q=%d kv=%d not supported (f32/f32, bf16/bf16, bf16/fp8_e4m3fn)",
                d.q_dtype, d.kv_dtype);
  if (d.max_blocks_per_seq <= 0)
    return fail(GQAP_ERR_INVALID_ARGUMENT, "max_blocks_per_seq must be positive (got %d)", d.max_blocks_per_seq);
  if (d.num_pool_blocks <= 0)
    return fail(GQAP_ERR_INVALID_ARGUMENT, "num_pool_blocks must be positive (got %d)", d.num_pool_blocks);
  if (d.max_seq_len < 0)
    return fail(GQAP_ERR_INVALID_ARGUMENT, "max_seq_len must be >= 0 (got %d)", d.max_seq_len);
  if ((int64_t)d.max_seq_len > (int64_t)d.max_blocks_per_seq * kBlock)
    return fail(GQAP_ERR_INVALID_ARGUMENT, "max_seq_len %d exceeds Nblk*64 = %lld", d.max_seq_len,
                (long long)d.max_blocks_per_seq * kBlock);
  const int64_t D = d.head_dim;
  if (d.q_stride_head < D || (d.num_q_heads > 1 && d.q_stride_batch < d.q_stride_head * d.num_q_heads))
    return fail(GQAP_ERR_INVALID_ARGUMENT, "q strides (batch %lld, head %lld) overlap for D=%lld",
                (long long)d.q_stride_batch, (long long)d.q_stride_head, (long long)D);
  if (d.num_q_heads == 1 && d.q_stride_batch < D)
    return fail(GQAP_ERR_INVALID_ARGUMENT, "q batch stride %lld < D", (long long)d.q_stride_batch);
  if (d.out_stride_head < D || (d.num_q_heads > 1 && d.out_stride_batch < d.out_stride_head * d.num_q_heads) ||
      (d.num_q_heads == 1 && d.out_stride_batch < D))
    return fail(GQAP_ERR_INVALID_ARGUMENT, "out strides (batch %lld, head %lld) overlap for D=%lld",
                (long long)d.out_stride_batch, (long long)d.out_stride_head, (long long)D);
  if (!aligned16(d.q_stride_head, *q_esz) || !aligned16(d.q_stride_batch, *q_esz) ||
      !aligned16(d.out_stride_head, *q_esz) || !aligned16(d.out_stride_batch, *q_esz))
    return fail(GQAP_ERR_INVALID_ARGUMENT, "q/out strides must keep rows 16-byte aligned");
  if (d.kv_stride_head < D * kBlock)
    return fail(GQAP_ERR_INVALID_ARGUMENT, "kv_stride_head %lld < 64*D: a (block, head) slab must be a contiguous 64 x D tile",
                (long long)d.kv_stride_head);
  if (d.kv_stride_block < d.kv_stride_head * d.num_kv_heads)
    return fail(GQAP_ERR_INVALID_ARGUMENT, "kv_stride_block %lld < Hk * kv_stride_head", (long long)d.kv_stride_block);
  if (!aligned16(d.kv_stride_head, *kv_esz) || !aligned16(d.kv_stride_block, *kv_esz))
    return fail(GQAP_ERR_INVALID_ARGUMENT, "kv strides must keep slabs 16-byte aligned");
  if (d.block_table_stride < d.max_blocks_per_seq)
    return fail(GQAP_ERR_INVALID_ARGUMENT, "block_table_stride %lld < Nblk %d", (long long)d.block_table_stride,
                d.max_blocks_per_seq);
  if (d.num_workers < 0 || d.num_workers > (1 << 20))
    return fail(GQAP_ERR_INVALID_ARGUMENT, "num_workers must be in [0, 2^20]");
  // The combine launches one 64-lane wave per (sequence, query head); a
  // launch holds fewer than 2^32 work-items.
  if ((int64_t)d.batch * d.num_q_heads * 64 > kMaxLaunchItems)
    return fail(GQAP_ERR_UNSUPPORTED, "batch * Hq = %lld (sequence, head) pairs exceed one combine launch",
                (long long)d.batch * d.num_q_heads);
  if (d.num_cus < 0) return fail(GQAP_ERR_INVALID_ARGUMENT, "num_cus must be >= 0");
  return GQAP_OK;
}

}  // namespace gqap

using namespace gqap;

extern "C" gqap_status gqap_decode_plan(const gqap_decode_desc_t* desc, gqap_decode_plan_t* plan) {
  if (!desc || !plan) return fail(GQAP_ERR_INVALID_ARGUMENT, "null desc or plan");
  std::memset(plan, 0, sizeof(*plan));
  int q_esz = 0, kv_esz = 0;
  gqap_status st = check_decode_desc(*desc, &q_esz, &kv_esz);
  if (st != GQAP_OK) return st;
  const gqap_decode_desc_t& d = *desc;
  plan->desc = d;
  plan->ratio = d.num_q_heads / d.num_kv_heads;
  plan->head_chunks = (int32_t)ceil_div(plan->ratio, 16);
  plan->kernel = d.kv_dtype == GQAP_F32 ? kDecodeF32Valu
                 : d.kv_dtype == GQAP_BF16 ? kDecodeBf16Mfma
                                            : kDecodeFp8Mfma;
  const int cus = d.num_cus ? d.num_cus : kDefaultCUs;
  plan->num_workers = d.num_workers > 0 ? d.num_workers : cus * decode_waves_per_cu(plan->kernel, d.head_dim);
  const int64_t pieces = (int64_t)d.batch * d.num_kv_heads * plan->head_chunks + plan->num_workers;
  if (pieces > INT32_MAX / 16) return fail(GQAP_ERR_INVALID_ARGUMENT, "too many partial slots");
  plan->max_pieces = (int32_t)pieces;
  plan->workspace_bytes = decode_workspace(d.batch, pieces, piece_cols(plan->ratio), d.head_dim).total;
  plan->magic = GQAP_PLAN_MAGIC;
  return GQAP_OK;
}

extern "C" gqap_status gqap_decode_validate_host(const gqap_decode_plan_t* plan, const int32_t* block_table_host,
                                                 const int32_t* seq_lens_host) {
  if (!plan || plan->magic != GQAP_PLAN_MAGIC) return fail(GQAP_ERR_INVALID_ARGUMENT, "invalid plan");
  const gqap_decode_desc_t& d = plan->desc;
  if (d.batch > 0 && (!block_table_host || !seq_lens_host))
    return fail(GQAP_ERR_INVALID_ARGUMENT, "null host metadata");
  const int64_t cap = std::min<int64_t>((int64_t)d.max_blocks_per_seq * kBlock, d.max_seq_len);
  for (int b = 0; b < d.batch; ++b) {
    const int64_t L = seq_lens_host[b];
    if (L < 0 || L > cap)
      return fail(GQAP_ERR_INVALID_ARGUMENT, "seq_lens[%d] = %lld outside [0, %lld]", b, (long long)L,
                  (long long)cap);
    const int64_t nb = ceil_div(L, kBlock);
    for (int64_t j = 0; j < nb; ++j) {
      const int64_t id = block_table_host[(int64_t)b * d.block_table_stride + j];
      if (id < 0 || id >= d.num_pool_blocks)
        return fail(GQAP_ERR_INVALID_ARGUMENT, "block_table[%d, %lld] = %lld outside the pool [0, %d)", b,
                    (long long)j, (long long)id, d.num_pool_blocks);
    }
  }
  return GQAP_OK;
}

// Key-axis splits of a prefill grid of `grid` workgroups (one per query tile
// and head).  Only a grid that leaves more than a quarter of the compute
// units without a workgroup is split: there the idle units are the loss.  A
// grid of one workgroup per unit or more is left alone, because the partial
// outputs a split writes and merges (fp32, 129 words per row and head) cost
// about what the second workgroup slot of a unit would gain.  The count
// fills the two slots of every unit, at most 4, and at most a quarter of the
// key tiles of the longest sequence (so every split keeps a few tiles to
// amortise its partial).  A positive request is taken as is.
static int32_t key_splits(int32_t requested, int64_t grid, int64_t max_keys, int32_t num_cus) {
  if (requested > 0) return requested;
  const int64_t cus = num_cus > 0 ? num_cus : 256;
  if (grid <= 0 || grid * 4 >= cus * 3) return 1;
  int64_t ns = std::min<int64_t>(4, ceil_div(2 * cus, grid));
  ns = std::min<int64_t>(ns, std::max<int64_t>(1, ceil_div(max_keys, kBlock) / 4));
  return (int32_t)std::max<int64_t>(1, ns);
}

static uint64_t split_workspace(int32_t ns, int64_t T, int64_t Hq) {
  return ns > 1 ? (uint64_t)ns * (uint64_t)T * (uint64_t)Hq * 129u * 4u : 0u;
}

extern "C" gqap_status gqap_prefill_plan(const gqap_prefill_desc_t* desc, gqap_prefill_plan_t* plan) {
  if (!desc || !plan) return fail(GQAP_ERR_INVALID_ARGUMENT, "null desc or plan");
  std::memset(plan, 0, sizeof(*plan));
  const gqap_prefill_desc_t& d = *desc;
  if (d.batch < 0) return fail(GQAP_ERR_INVALID_ARGUMENT, "batch must be >= 0");
  if (d.num_q_heads <= 0 || d.num_kv_heads <= 0)
    return fail(GQAP_ERR_INVALID_ARGUMENT, "head counts must be positive (Hq=%d, Hk=%d)", d.num_q_heads,
                d.num_kv_heads);
  if (d.num_q_heads % d.num_kv_heads)
    return fail(GQAP_ERR_INVALID_ARGUMENT, "Hq (%d) must be a multiple of Hk (%d)", d.num_q_heads, d.num_kv_heads);
  if (d.dtype != GQAP_BF16 && d.dtype != GQAP_FP8_E4M3FN)
    return fail(GQAP_ERR_DTYPE, "prefill takes bf16, or fp8 q_nope/k (got dtype %d)", d.dtype);
  const bool f8 = d.dtype == GQAP_FP8_E4M3FN;
  if (d.causal != 1) return fail(GQAP_ERR_UNSUPPORTED, "only causal prefill is implemented");
  const bool mla = d.head_dim_qk == 192 && d.head_dim_rope == 64;
  const bool plain = d.head_dim_qk == 128 && d.head_dim_rope == 0;
  if (!mla && !plain)
    return fail(GQAP_ERR_UNSUPPORTED, "head widths qk=%d rope=%d not supported (128/0 or 192/64)", d.head_dim_qk,
                d.head_dim_rope);
  if (d.head_dim_v != 128) return fail(GQAP_ERR_UNSUPPORTED, "head_dim_v must be 128 (got %d)", d.head_dim_v);
  if (d.total_tokens < 0 || d.max_seq_len < 0)
    return fail(GQAP_ERR_INVALID_ARGUMENT, "total_tokens and max_seq_len must be >= 0");
  if (d.max_seq_len > d.total_tokens && d.batch > 0)
    return fail(GQAP_ERR_INVALID_ARGUMENT, "max_seq_len %d exceeds total_tokens %d", d.max_seq_len, d.total_tokens);
  const int64_t Dn = d.head_dim_qk - d.head_dim_rope;
  // fp8: q holds the nope part only, the rope part is the bf16 tensor q_rope.
  if (d.q_stride_head < (f8 ? Dn : d.head_dim_qk) || d.q_stride_token < d.q_stride_head * d.num_q_heads)
    return fail(GQAP_ERR_INVALID_ARGUMENT, "q strides overlap");
  if (f8 && d.head_dim_rope &&
      (d.qr_stride_head < d.head_dim_rope || d.qr_stride_token < d.qr_stride_head * d.num_q_heads))
    return fail(GQAP_ERR_INVALID_ARGUMENT, "q_rope strides overlap");
  if (d.k_stride_head < Dn || d.k_stride_token < d.k_stride_head * d.num_kv_heads)
    return fail(GQAP_ERR_INVALID_ARGUMENT, "k strides overlap");
  if (d.v_stride_head < d.head_dim_v || d.v_stride_token < d.v_stride_head * d.num_kv_heads)
    return fail(GQAP_ERR_INVALID_ARGUMENT, "v strides overlap");
  if (d.out_stride_head < d.head_dim_v || d.out_stride_token < d.out_stride_head * d.num_q_heads)
    return fail(GQAP_ERR_INVALID_ARGUMENT, "out strides overlap");
  if (d.head_dim_rope && d.kr_stride_token < d.head_dim_rope)
    return fail(GQAP_ERR_INVALID_ARGUMENT, "k_rope token stride < rope width");
  const int64_t strides[] = {d.v_stride_token, d.v_stride_head, d.out_stride_token, d.out_stride_head,
                             d.head_dim_rope ? d.kr_stride_token : 8,
                             f8 && d.head_dim_rope ? d.qr_stride_token : 8, f8 && d.head_dim_rope ? d.qr_stride_head : 8};
  const int64_t qk_strides[] = {d.q_stride_token, d.q_stride_head, d.k_stride_token, d.k_stride_head};
  bool ok = true;
  for (int64_t s : strides) ok = ok && aligned16(s, 2);
  for (int64_t s : qk_strides) ok = ok && aligned16(s, f8 ? 1 : 2);
  if (!ok) return fail(GQAP_ERR_INVALID_ARGUMENT, "strides must keep rows 16-byte aligned");
  if (d.has_block_mask != 0 && d.has_block_mask != 1)
    return fail(GQAP_ERR_INVALID_ARGUMENT, "has_block_mask must be 0 or 1");
  if (d.has_block_mask && (int64_t)d.mask_blocks < ceil_div(d.max_seq_len, kBlock))
    return fail(GQAP_ERR_INVALID_ARGUMENT, "mask_blocks %d < ceil(max_seq_len/64)", d.mask_blocks);
  if (d.num_cus < 0) return fail(GQAP_ERR_INVALID_ARGUMENT, "num_cus must be >= 0");
  if (d.num_splits < 0 || d.num_splits > 16)
    return fail(GQAP_ERR_INVALID_ARGUMENT, "num_splits must be 0 (automatic) or 1..16 (got %d)", d.num_splits);
  plan->desc = d;
  plan->ratio = d.num_q_heads / d.num_kv_heads;
  // A workgroup takes 128 query rows of one head, or, with a block mask and
  // heads of a KV group that pair up (Hq / Hk even), 64 rows of two heads of
  // the group: its two 64-row query blocks would follow different mask rows,
  // and half its waves would sit out every tile only one block needs, while
  // the two heads of a pair follow the same row.  Without a mask the two
  // blocks see nearly the same tiles and 128-row tiles measure faster.
  plan->q_tile_rows = plan->ratio % 2 == 0 && d.has_block_mask ? 64 : 128;
  // At least one query tile per sequence, so that a sequence longer than the
  // capacity always has a workgroup to clear its rows past max_seq_len.
  plan->q_tiles = (int32_t)std::max<int64_t>(d.batch > 0 ? 1 : 0, ceil_div(d.max_seq_len, plan->q_tile_rows));
  const int64_t grid = (int64_t)d.num_q_heads * d.batch * plan->q_tiles * plan->q_tile_rows / 128;
  const int32_t ns = key_splits(d.num_splits, grid, d.max_seq_len, d.num_cus);
  // One workgroup of 256 work-items per (head, sequence, query tile, split)
  // slot; the launch must stay under 2^32 work-items.
  if (grid * ns >= ((int64_t)1 << 24))
    return fail(GQAP_ERR_UNSUPPORTED,
                "Hq * batch * ceil(max_seq_len/128) * num_splits = %lld workgroups exceeds 2^24",
                (long long)(grid * ns));
  // The split merge runs at most one 64-lane wave per (token, head).
  if (ns > 1 && (int64_t)d.total_tokens * d.num_q_heads * 64 > kMaxLaunchItems)
    return fail(GQAP_ERR_UNSUPPORTED, "T * Hq = %lld (token, head) pairs exceed one split-merge launch",
                (long long)d.total_tokens * d.num_q_heads);
  plan->kernel = (mla ? 2 : 1) + (f8 ? 2 : 0);
  plan->num_splits = (uint32_t)ns;
  plan->workspace_bytes = split_workspace(ns, d.total_tokens, d.num_q_heads);
  plan->magic = GQAP_PLAN_MAGIC;
  return GQAP_OK;
}

// Chunked prefill against the paged cache (FlashMLA tensor-shape reference,
// section 4: a prefill with a KV cache writes into 64-row pages).  The same
// shape rules as decode for the cache, ragged token-major rows for the chunk.
extern "C" gqap_status gqap_chunk_plan(const gqap_chunk_desc_t* desc, gqap_chunk_plan_t* plan) {
  if (!desc || !plan) return fail(GQAP_ERR_INVALID_ARGUMENT, "null desc or plan");
  std::memset(plan, 0, sizeof(*plan));
  const gqap_chunk_desc_t& d = *desc;
  if (d.batch < 0) return fail(GQAP_ERR_INVALID_ARGUMENT, "batch must be >= 0");
  if (d.num_q_heads <= 0 || d.num_kv_heads <= 0)
    return fail(GQAP_ERR_INVALID_ARGUMENT, "head counts must be positive (Hq=%d, Hk=%d)", d.num_q_heads,
                d.num_kv_heads);
  if (d.num_q_heads % d.num_kv_heads)
    return fail(GQAP_ERR_INVALID_ARGUMENT, "Hq (%d) must be a multiple of Hk (%d)", d.num_q_heads, d.num_kv_heads);
  if (d.block_size != kBlock) return fail(GQAP_ERR_UNSUPPORTED, "block_size must be %d (got %d)", kBlock, d.block_size);
  if (d.head_dim != 128) return fail(GQAP_ERR_UNSUPPORTED, "head_dim must be 128 (got %d)", d.head_dim);
  if (d.dtype != GQAP_BF16) return fail(GQAP_ERR_DTYPE, "chunked prefill takes bf16 tensors (got dtype %d)", d.dtype);
  // The cache: bf16 like the chunk (kv_dtype 0 in a zero-filled descriptor),
  // or fp8 e4m3fn codes with per-tensor scales.
  if (d.kv_dtype != 0 && d.kv_dtype != GQAP_BF16 && d.kv_dtype != GQAP_FP8_E4M3FN)
    return fail(GQAP_ERR_DTYPE, "kv_dtype must be 0, GQAP_BF16 or GQAP_FP8_E4M3FN (got %d)", d.kv_dtype);
  const int kv_esz = d.kv_dtype == GQAP_FP8_E4M3FN ? 1 : 2;
  if (d.max_blocks_per_seq <= 0)
    return fail(GQAP_ERR_INVALID_ARGUMENT, "max_blocks_per_seq must be positive (got %d)", d.max_blocks_per_seq);
  if (d.num_pool_blocks <= 0)
    return fail(GQAP_ERR_INVALID_ARGUMENT, "num_pool_blocks must be positive (got %d)", d.num_pool_blocks);
  if (d.total_q_tokens < 0 || d.max_q_len < 0 || d.max_kv_len < 0)
    return fail(GQAP_ERR_INVALID_ARGUMENT, "total_q_tokens, max_q_len and max_kv_len must be >= 0");
  if ((int64_t)d.max_kv_len > (int64_t)d.max_blocks_per_seq * kBlock)
    return fail(GQAP_ERR_INVALID_ARGUMENT, "max_kv_len %d exceeds Nblk*64 = %lld", d.max_kv_len,
                (long long)d.max_blocks_per_seq * kBlock);
  if (d.max_q_len > d.max_kv_len)
    return fail(GQAP_ERR_INVALID_ARGUMENT, "max_q_len %d exceeds max_kv_len %d (a chunk's tokens are among its keys)",
                d.max_q_len, d.max_kv_len);
  if (d.head_dim_rope != 0 && d.head_dim_rope != 64)
    return fail(GQAP_ERR_UNSUPPORTED, "head_dim_rope must be 0 or 64 (got %d)", d.head_dim_rope);
  const int64_t D = d.head_dim, Dr = d.head_dim_rope, Hq = d.num_q_heads, Hk = d.num_kv_heads;
  if (d.q_stride_head < D + Dr || d.q_stride_token < d.q_stride_head * Hq)
    return fail(GQAP_ERR_INVALID_ARGUMENT, "q strides overlap");
  if (Dr && (d.kr_new_stride_token < Dr || d.kr_stride_block < Dr * kBlock || !aligned16(d.kr_new_stride_token, 2) ||
             !aligned16(d.kr_stride_block, 2)))
    return fail(GQAP_ERR_INVALID_ARGUMENT, "rope strides (new %lld, block %lld) overlap or break 16-byte alignment",
                (long long)d.kr_new_stride_token, (long long)d.kr_stride_block);
  if (d.new_stride_head < D || d.new_stride_token < d.new_stride_head * Hk)
    return fail(GQAP_ERR_INVALID_ARGUMENT, "k_new/v_new strides overlap");
  if (d.out_stride_head < D || d.out_stride_token < d.out_stride_head * Hq)
    return fail(GQAP_ERR_INVALID_ARGUMENT, "out strides overlap");
  if (d.kv_stride_head < D * kBlock)
    return fail(GQAP_ERR_INVALID_ARGUMENT, "kv_stride_head %lld < 64*D: a (block, head) slab must be a contiguous 64 x D tile",
                (long long)d.kv_stride_head);
  if (d.kv_stride_block < d.kv_stride_head * Hk)
    return fail(GQAP_ERR_INVALID_ARGUMENT, "kv_stride_block %lld < Hk * kv_stride_head", (long long)d.kv_stride_block);
  if (d.block_table_stride < d.max_blocks_per_seq)
    return fail(GQAP_ERR_INVALID_ARGUMENT, "block_table_stride %lld < Nblk %d", (long long)d.block_table_stride,
                d.max_blocks_per_seq);
  const int64_t strides[] = {d.q_stride_token, d.q_stride_head, d.new_stride_token, d.new_stride_head,
                             d.out_stride_token, d.out_stride_head};
  for (int64_t st : strides)
    if (!aligned16(st, 2)) return fail(GQAP_ERR_INVALID_ARGUMENT, "strides must keep rows 16-byte aligned");
  if (!aligned16(d.kv_stride_block, kv_esz) || !aligned16(d.kv_stride_head, kv_esz))
    return fail(GQAP_ERR_INVALID_ARGUMENT, "pool strides must keep page slabs 16-byte aligned");
  plan->desc = d;
  plan->ratio = d.num_q_heads / d.num_kv_heads;
  plan->q_tile_rows = 128;  // no block mask: one head per workgroup
  // At least one query tile per sequence (see the prefill plan).
  plan->q_tiles = (int32_t)std::max<int64_t>(d.batch > 0 ? 1 : 0, ceil_div(d.max_q_len, plan->q_tile_rows));
  if (d.num_splits < 0 || d.num_splits > 16)
    return fail(GQAP_ERR_INVALID_ARGUMENT, "num_splits must be 0 (automatic) or 1..16 (got %d)", d.num_splits);
  const int64_t grid = (int64_t)d.num_q_heads * d.batch * plan->q_tiles * plan->q_tile_rows / 128;
  const int32_t ns = key_splits(d.num_splits, grid, d.max_kv_len, 0);
  // One workgroup of 256 work-items per (head, sequence, query tile) slot;
  // the launch must stay under 2^32 work-items.
  if (grid * ns >= ((int64_t)1 << 24))
    return fail(GQAP_ERR_UNSUPPORTED, "Hq * batch * ceil(max_q_len/128) * num_splits = %lld workgroups exceeds 2^24",
                (long long)(grid * ns));
  if (ns > 1 && (int64_t)d.total_q_tokens * Hq * 64 > kMaxLaunchItems)
    return fail(GQAP_ERR_UNSUPPORTED, "T * Hq = %lld (token, head) pairs exceed one split-merge launch",
                (long long)d.total_q_tokens * Hq);
  // The append runs one work-item per 16-byte piece of a (token, KV head) row.
  if ((int64_t)d.total_q_tokens * Hk * (D / 8) > kMaxLaunchItems)
    return fail(GQAP_ERR_UNSUPPORTED, "T * Hk = %lld (token, KV head) rows exceed one append launch",
                (long long)d.total_q_tokens * Hk);
  plan->kernel = (Dr ? kChunkPrefillMla : kChunkPrefill) + (kv_esz == 1 ? 2 : 0);
  plan->num_splits = (uint32_t)ns;
  plan->workspace_bytes = split_workspace(ns, d.total_q_tokens, d.num_q_heads);
  // Short chunks go to the decode workers when the (token, head) pairs of a
  // KV head fit in as many 16-column tiles as one token's heads: every K/V
  // byte is then read once per tile, where the prefill kernel reads it once
  // per query head.  With the MLA rope cache every query head's tiles also
  // read the shared rope rows.  Forced splits keep the prefill kernel.
  const int64_t hc_token = ceil_div(plan->ratio, 16);
  const int64_t hc_chunk = ceil_div((int64_t)d.max_q_len * plan->ratio, 16);
  if (d.num_splits == 0 && d.max_q_len >= 1 && hc_chunk == hc_token) {
    plan->kernel = kv_esz == 1 ? kChunkDecodeFp8 : kChunkDecode;
    plan->num_splits = 1;
    plan->head_chunks = (int32_t)hc_chunk;
    plan->num_workers = kDefaultCUs * decode_waves_per_cu(kv_esz == 1 ? kDecodeFp8Mfma : kDecodeBf16Mfma, 128);
    const int64_t pieces = (int64_t)d.batch * Hk * hc_chunk + plan->num_workers;
    if (pieces > INT32_MAX / 16) return fail(GQAP_ERR_UNSUPPORTED, "too many partial slots for the decode workers");
    plan->workspace_bytes =
        decode_workspace(d.batch, pieces, piece_cols((int64_t)d.max_q_len * plan->ratio), D).total;
  }
  plan->magic = GQAP_PLAN_MAGIC;
  return GQAP_OK;
}

extern "C" gqap_status gqap_chunk_validate_host(const gqap_chunk_plan_t* plan, const int32_t* block_table_host,
                                                const int32_t* cu_seqlens_q_host, const int32_t* kv_lens_host) {
  if (!plan || plan->magic != GQAP_PLAN_MAGIC) return fail(GQAP_ERR_INVALID_ARGUMENT, "invalid plan");
  const gqap_chunk_desc_t& d = plan->desc;
  if (!cu_seqlens_q_host || (d.batch > 0 && (!block_table_host || !kv_lens_host)))
    return fail(GQAP_ERR_INVALID_ARGUMENT, "null host metadata");
  if (cu_seqlens_q_host[0] != 0) return fail(GQAP_ERR_INVALID_ARGUMENT, "cu_seqlens_q[0] = %d, not 0", cu_seqlens_q_host[0]);
  for (int b = 0; b < d.batch; ++b) {
    const int64_t ql = (int64_t)cu_seqlens_q_host[b + 1] - cu_seqlens_q_host[b];
    const int64_t kl = kv_lens_host[b];
    if (ql < 0 || cu_seqlens_q_host[b + 1] > d.total_q_tokens)
      return fail(GQAP_ERR_INVALID_ARGUMENT, "cu_seqlens_q[%d..%d] = %d..%d decreases or passes T = %d", b, b + 1,
                  cu_seqlens_q_host[b], cu_seqlens_q_host[b + 1], d.total_q_tokens);
    if (ql > d.max_q_len)
      return fail(GQAP_ERR_INVALID_ARGUMENT, "chunk %d has %lld tokens > max_q_len %d", b, (long long)ql, d.max_q_len);
    if (kl < ql || kl > d.max_kv_len)
      return fail(GQAP_ERR_INVALID_ARGUMENT, "kv_lens[%d] = %lld outside [q_len %lld, max_kv_len %d]", b,
                  (long long)kl, (long long)ql, d.max_kv_len);
    for (int64_t j = 0; j < ceil_div(kl, kBlock); ++j) {
      const int64_t id = block_table_host[(int64_t)b * d.block_table_stride + j];
      if (id < 0 || id >= d.num_pool_blocks)
        return fail(GQAP_ERR_INVALID_ARGUMENT, "block_table[%d, %lld] = %lld outside the pool [0, %d)", b,
                    (long long)j, (long long)id, d.num_pool_blocks);
    }
  }
  return GQAP_OK;
}

extern "C" const char* gqap_last_error(void) { return last_error_slot().c_str(); }

extern "C" const char* gqap_version(void) { return "gqap 0.1.0 (gfx950)"; }
